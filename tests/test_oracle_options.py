"""Pins of the oracle's general top-K loss (``topk_loss_*``): the partial-mass
teacher, per-token temperature, the LM cross-entropy mix and KL mixing over the
cached entries; and of the full-vocabulary KL mixing.  CPU only.

Sources: "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a
Fused Chunked KL Loss", §3 "Offline distillation" (cached probabilities keep
their unnormalised partial mass; teacher-entropy, cross and mass terms over
the support, plus the one full-vocabulary log Z) and "Offline
implementations" (the dense reconstruction is the correctness baseline); the
adaptive-distillation abstract on the WASD page (per-token temperature); the
teacher-strength abstract (mixing the LM and KD losses); the KL-direction
abstract (forward and reverse token-level KL and their mixture).  Every pin checks the
oracle against something other than its own formula: a library routine, an
identity that relates it to the already pinned renormalised oracle, autograd
of the dense reconstruction, or finite differences.
"""
import numpy as np
import pytest
import scipy.special as sps
import torch

from oracle import kd_oracle as O


def case(T=6, d=8, V=32, K=5, seed=0, dup=False):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((d, V)) / np.sqrt(d)
    A = -np.sort(-rng.standard_normal((T, K)) * 1.7, axis=1)
    I = np.stack([rng.choice(V, K, replace=False) for _ in range(T)]).astype(np.int64)
    if dup:
        I[:, 1] = I[:, 0]
    g = rng.standard_normal(T)
    taus = rng.uniform(0.6, 2.5, T)
    y = rng.integers(0, V, T)
    return H, W, I, A, g, taus, y


def teacher_lse_for_mass(A, taus, rng):
    """A per-row log-normaliser that leaves mass m_t in (0.15, 0.95) on the K entries."""
    a = A / taus[:, None]
    m = rng.uniform(0.15, 0.95, A.shape[0])
    return sps.logsumexp(a, axis=1) - np.log(m), m


# ---------------------------------------------------------------- partial mass
def test_partial_mass_with_every_entry_is_torch_kl_div():
    # K = V, the full teacher softmax cached (teacher_lse its true log Z):
    # the support identity must equal the full-vocabulary KL of torch
    rng = np.random.default_rng(1)
    T, d, V = 5, 8, 24
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((d, V)) / np.sqrt(d)
    U = rng.standard_normal((T, V)) * 2.0
    I = np.stack([rng.permutation(V) for _ in range(T)])
    A = np.take_along_axis(U, I, axis=1)
    for tau in (1.0, 1.7):
        tl = sps.logsumexp(U / tau, axis=1)
        got, _, _ = O.topk_loss_forward(H, W, I, A, None, tau, teacher_lse=tl)
        logq = torch.log_softmax(torch.tensor(H @ W) / tau, dim=1)
        logp = torch.log_softmax(torch.tensor(U) / tau, dim=1)
        want = torch.nn.functional.kl_div(logq, logp, log_target=True, reduction="none").sum(1).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_partial_mass_scaling_identity():
    # p = m p~ with p~ the renormalised teacher: KD = m (KL_renormalised + log m)
    H, W, I, A, g, _, _ = case(T=8, seed=2)
    rng = np.random.default_rng(3)
    for tau in (1.0, 0.7, 2.2):
        tl, m = teacher_lse_for_mass(A, np.full(8, tau), rng)
        got, lse, _ = O.topk_loss_forward(H, W, I, A, None, tau, teacher_lse=tl)
        ren, lse2, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        np.testing.assert_allclose(got, m * (ren + np.log(m)), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, lse2, rtol=1e-14)


def _dense_partial_mass(Ht, Wt, I, A, tl, taus, g):
    """Dense reconstruction ([EKD] §3 "Offline implementations") with the
    cached probabilities scattered unnormalised into a [T, V] tensor."""
    T, V = Ht.shape[0], Wt.shape[1]
    tau = torch.tensor(taus)[:, None]
    logq = torch.log_softmax((Ht @ Wt) / tau, dim=1)
    p = torch.exp(torch.tensor(A) / tau - torch.tensor(tl)[:, None])
    P = torch.zeros(T, V, dtype=torch.float64).scatter_add_(1, torch.tensor(I), p)
    plogp = torch.where(P > 0, P * torch.log(torch.where(P > 0, P, torch.ones_like(P))), torch.zeros_like(P))
    kd = (plogp - P * logq).sum(1)
    return (kd * torch.tensor(g)).sum(), kd


def test_partial_mass_matches_autograd_of_dense_reconstruction():
    H, W, I, A, g, taus, _ = case(T=7, d=6, V=25, seed=4)
    rng = np.random.default_rng(5)
    tl, _ = teacher_lse_for_mass(A, taus, rng)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss, kd = _dense_partial_mass(Ht, Wt, I, A, tl, taus, g)
    loss.backward()
    got, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, teacher_lse=tl)
    np.testing.assert_allclose(got, kd.detach().numpy(), rtol=1e-12)
    dH, dW = O.topk_loss_backward(H, W, I, A, None, 1.0, g, tau_rows=taus, teacher_lse=tl)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_partial_mass_gradient_rows_sum_to_zero():
    # sum_v dZ_tv = (g_t / tau_t) (m_t - m_t) = 0 for KD alone: the mass term
    # of the gradient (m q) balances the scattered p exactly, so dW . 1 = 0
    H, W, I, A, g, taus, _ = case(T=6, seed=6)
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(7))
    _, dW = O.topk_loss_backward(H, W, I, A, None, 1.0, g, tau_rows=taus, teacher_lse=tl)
    np.testing.assert_allclose(dW.sum(1), 0.0, atol=1e-13)


# ---------------------------------------------------------------- per-token temperature
def test_per_token_tau_is_row_scaling():
    # row t at tau_t equals the tau = 1 loss of (H_t / tau_t, A_t / tau_t)
    H, W, I, A, g, taus, _ = case(T=7, seed=8)
    got, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus)
    want, _, _ = O.topk_kl_forward(H / taus[:, None], W, I, A / taus[:, None], None, 1.0)
    np.testing.assert_allclose(got, want, rtol=1e-12)
    # one row at a time through the scalar-tau oracle
    for t in range(7):
        one, _, _ = O.topk_kl_forward(H[t:t + 1], W, I[t:t + 1], A[t:t + 1], None, taus[t])
        assert got[t] == pytest.approx(one[0], rel=1e-12)


def test_per_token_tau_gradient_is_row_scaled_plain_gradient():
    # dH_t at tau_t equals the plain oracle's dH of (H_t / tau_t, A_t / tau_t) at
    # tau = 1, divided by tau_t (chain rule through H / tau_t)
    H, W, I, A, g, taus, _ = case(T=6, seed=9)
    dH, _ = O.topk_loss_backward(H, W, I, A, None, 1.0, g, tau_rows=taus)
    dH1, _ = O.topk_kl_backward(H / taus[:, None], W, I, A / taus[:, None], None, 1.0, g)
    np.testing.assert_allclose(dH, dH1 / taus[:, None], rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- LM cross-entropy mix
def test_ce_weight_one_is_torch_cross_entropy():
    H, W, I, A, g, taus, y = case(T=9, V=40, seed=10)
    got, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, labels=y, ce_weight=1.0)
    logits = torch.tensor(H @ W) / torch.tensor(taus)[:, None]
    want = torch.nn.functional.cross_entropy(logits, torch.tensor(y), reduction="none").numpy()
    np.testing.assert_allclose(got, want, rtol=1e-13)


def test_ce_mix_is_the_convex_combination():
    H, W, I, A, g, _, y = case(T=8, V=36, seed=11)
    for tau, beta in ((1.0, 0.25), (1.6, 0.5), (0.8, 0.9)):
        got, lse, _ = O.topk_loss_forward(H, W, I, A, None, tau, labels=y, ce_weight=beta)
        kd, lse2, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        ce = torch.nn.functional.cross_entropy(torch.tensor(H @ W / tau), torch.tensor(y),
                                               reduction="none").numpy()
        np.testing.assert_allclose(got, (1 - beta) * kd + beta * ce, rtol=1e-12)
        np.testing.assert_allclose(lse, lse2, rtol=1e-14)


def test_ce_gradient_matches_torch_autograd():
    H, W, I, A, g, _, y = case(T=6, V=30, seed=12)
    tau, beta = 1.3, 0.4
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    logits = Ht @ Wt / tau
    ce = torch.nn.functional.cross_entropy(logits, torch.tensor(y), reduction="none")
    (beta * ce * torch.tensor(g)).sum().backward()
    dH_ce, dW_ce = Ht.grad.numpy().copy(), Wt.grad.numpy().copy()
    dH_kd, dW_kd = O.topk_kl_backward(H, W, I, A, None, tau, g)
    dH, dW = O.topk_loss_backward(H, W, I, A, None, tau, g, labels=y, ce_weight=beta)
    np.testing.assert_allclose(dH, (1 - beta) * dH_kd + dH_ce, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, (1 - beta) * dW_kd + dW_ce, rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- all options at once
def test_all_options_finite_differences():
    H, W, I, A, g, taus, y = case(T=4, d=8, V=32, K=4, seed=13, dup=True)
    y[0] = I[0, 2]  # a label that is also a cached index
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(14))
    mask = np.array([1, 0, 1, 1], dtype=np.uint8)
    kw = dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=0.35)
    dH, dW = O.topk_loss_backward(H, W, I, A, mask, 1.0, g, **kw)

    def loss(Hx, Wx):
        v, _, _ = O.topk_loss_forward(Hx, Wx, I, A, mask, 1.0, **kw)
        return float((v * g).sum())

    h = 1e-6
    rng = np.random.default_rng(15)
    for _ in range(12):
        t, j = rng.integers(4), rng.integers(8)
        Hp, Hm = H.copy(), H.copy()
        Hp[t, j] += h
        Hm[t, j] -= h
        assert (loss(Hp, W) - loss(Hm, W)) / (2 * h) == pytest.approx(dH[t, j], rel=1e-7, abs=1e-9)
    for _ in range(12):
        j, v = rng.integers(8), rng.integers(32)
        Wp, Wm = W.copy(), W.copy()
        Wp[j, v] += h
        Wm[j, v] -= h
        assert (loss(H, Wp) - loss(H, Wm)) / (2 * h) == pytest.approx(dW[j, v], rel=1e-7, abs=1e-9)
    assert np.all(dH[1] == 0)


def test_no_options_is_the_plain_loss():
    H, W, I, A, g, _, _ = case(T=7, seed=16)
    a = O.topk_loss_forward(H, W, I, A, None, 1.4)
    b = O.topk_kl_forward(H, W, I, A, None, 1.4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(O.topk_loss_backward(H, W, I, A, None, 1.4, g)[1],
                               O.topk_kl_backward(H, W, I, A, None, 1.4, g)[1], rtol=1e-12, atol=1e-15)


def test_masked_rows_ignore_garbage_options():
    H, W, I, A, g, taus, y = case(T=5, seed=17)
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(18))
    mask = np.array([1, 0, 1, 0, 1], dtype=np.uint8)
    taus[1], tl[3], y[1], y[3] = np.nan, np.nan, -7, 10 ** 6
    H[3] = np.nan
    kw = dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=0.5)
    v, lse, z = O.topk_loss_forward(H, W, I, A, mask, 1.0, **kw)
    dH, dW = O.topk_loss_backward(H, W, I, A, mask, 1.0, g, **kw)
    assert np.all(v[[1, 3]] == 0) and np.all(lse[[1, 3]] == 0) and np.all(dH[[1, 3]] == 0)
    assert np.all(np.isfinite(v)) and np.all(np.isfinite(dW))


def test_rows_helper_matches_full_functions():
    H, W, I, A, g, taus, y = case(T=9, seed=19)
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(20))
    kw = dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=0.3, rev_weight=0.4)
    v, lse, z = O.topk_loss_forward(H, W, I, A, None, 1.0, **kw)
    dH, _ = O.topk_loss_backward(H, W, I, A, None, 1.0, g, **kw)
    rows = [0, 4, 8]
    rv, rl, rz, rdH = O.topk_loss_rows(H, W, I, A, None, 1.0, g, rows, **kw)
    np.testing.assert_allclose(rv, v[rows], rtol=1e-14)
    np.testing.assert_allclose(rdH, dH[rows], rtol=1e-13, atol=1e-16)


# ---------------------------------------------------------------- top-K: KL mixing over the cached entries
def _torch_support_kls(H, W, I, A, taus):
    """Forward and reverse KL between the student and the teacher restricted
    to the K cached entries and renormalised there, with torch's kl_div."""
    tau = torch.tensor(taus)[:, None]
    a = torch.gather(torch.tensor(H @ W) / tau, 1, torch.tensor(I))
    logq = torch.log_softmax(a, dim=1)
    logp = torch.log_softmax(torch.tensor(A) / tau, dim=1)
    rev = torch.nn.functional.kl_div(logp, logq, log_target=True, reduction="none").sum(1).numpy()
    fwd = torch.nn.functional.kl_div(logq, logp, log_target=True, reduction="none").sum(1).numpy()
    return fwd, rev


def test_topk_reverse_with_every_entry_is_the_full_vocab_reverse():
    # K = V (a permutation of the vocabulary per row): the cached entries are
    # the whole vocabulary, so the mixed top-K loss and its gradient must be
    # the full-vocabulary mixed loss of a teacher whose logits are U (teacher
    # head = identity, its hidden state = U), itself pinned to torch above
    rng = np.random.default_rng(40)
    T, d, V = 5, 7, 18
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((d, V)) / np.sqrt(d)
    U = rng.standard_normal((T, V)) * 1.8
    I = np.stack([rng.permutation(V) for _ in range(T)])
    A = np.take_along_axis(U, I, axis=1)
    g = rng.standard_normal(T)
    taus = rng.uniform(0.7, 2.0, T)
    for r in (0.0, 0.35, 1.0):
        got = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, rev_weight=r)
        want = O.full_loss_forward(H, W, U, np.eye(V), None, 1.0, tau_rows=taus, rev_weight=r)
        np.testing.assert_allclose(got[0], want[0], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-13)
        dH, dW = O.topk_loss_backward(H, W, I, A, None, 1.0, g, tau_rows=taus, rev_weight=r)
        fH, fW = O.full_loss_backward(H, W, U, np.eye(V), None, 1.0, g, tau_rows=taus, rev_weight=r)
        np.testing.assert_allclose(dH, fH, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(dW, fW, rtol=1e-10, atol=1e-13)


def test_topk_reverse_is_torch_kl_div_on_the_support():
    # r = 1: the loss is KL(q~ || p^) over the K entries; the partial mass
    # leaves it unchanged (both sides are renormalised on the support)
    H, W, I, A, g, taus, _ = case(T=8, V=40, K=6, seed=41, dup=True)
    fwd, rev = _torch_support_kls(H, W, I, A, taus)
    got, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, rev_weight=1.0)
    np.testing.assert_allclose(got, rev, rtol=1e-12, atol=1e-14)
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(42))
    got2, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, teacher_lse=tl, rev_weight=1.0)
    np.testing.assert_allclose(got2, rev, rtol=1e-12, atol=1e-14)
    assert np.all(rev >= 0) and np.all(np.abs(rev - fwd) > 1e-6)  # the two directions differ here
    # mixing: the convex combination with the (already pinned) forward-KL loss
    kd, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, teacher_lse=tl)
    for r in (0.2, 0.7):
        mix, _, _ = O.topk_loss_forward(H, W, I, A, None, 1.0, tau_rows=taus, teacher_lse=tl, rev_weight=r)
        np.testing.assert_allclose(mix, (1 - r) * kd + r * rev, rtol=1e-12, atol=1e-14)


def test_topk_mixed_gradient_matches_torch_autograd():
    # every option at once, duplicates and a masked row, against autograd of
    # the loss written with torch's log_softmax, kl_div and cross_entropy
    H, W, I, A, g, taus, y = case(T=6, d=7, V=30, K=5, seed=43, dup=True)
    y[2] = I[2, 3]
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(44))
    mask = np.array([1, 1, 0, 1, 1, 1], dtype=np.uint8)
    for r, beta in ((0.5, 0.0), (0.3, 0.25), (1.0, 0.6)):
        Hv = torch.tensor(H, requires_grad=True)
        Wv = torch.tensor(W, requires_grad=True)
        tau = torch.tensor(taus)[:, None]
        s = (Hv @ Wv) / tau
        logq = torch.log_softmax(s, dim=1)
        p = torch.exp(torch.tensor(A) / tau - torch.tensor(tl)[:, None])
        kd = (p * torch.log(p)).sum(1) - (p * torch.gather(logq, 1, torch.tensor(I))).sum(1)
        lqs = torch.log_softmax(torch.gather(s, 1, torch.tensor(I)), dim=1)
        lps = torch.log_softmax(torch.tensor(A) / tau, dim=1)
        rkl = torch.nn.functional.kl_div(lps, lqs, log_target=True, reduction="none").sum(1)
        ce = torch.nn.functional.cross_entropy(s, torch.tensor(y), reduction="none")
        loss = (1 - beta) * ((1 - r) * kd + r * rkl) + beta * ce
        m = torch.tensor(mask, dtype=torch.float64)
        (loss * m * torch.tensor(g)).sum().backward()
        kw = dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=beta, rev_weight=r)
        got, _, _ = O.topk_loss_forward(H, W, I, A, mask, 1.0, **kw)
        np.testing.assert_allclose(got, (loss * m).detach().numpy(), rtol=1e-11, atol=1e-13)
        dH, dW = O.topk_loss_backward(H, W, I, A, mask, 1.0, g, **kw)
        np.testing.assert_allclose(dH, Hv.grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(dW, Wv.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_topk_reverse_finite_differences():
    H, W, I, A, g, taus, y = case(T=4, d=8, V=32, K=4, seed=45, dup=True)
    tl, _ = teacher_lse_for_mass(A, taus, np.random.default_rng(46))
    mask = np.array([1, 1, 0, 1], dtype=np.uint8)
    kw = dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=0.2, rev_weight=0.65)
    dH, dW = O.topk_loss_backward(H, W, I, A, mask, 1.0, g, **kw)

    def loss(Hx, Wx):
        v, _, _ = O.topk_loss_forward(Hx, Wx, I, A, mask, 1.0, **kw)
        return float((v * g).sum())

    h = 1e-6
    rng = np.random.default_rng(47)
    for _ in range(10):
        t, j = rng.integers(4), rng.integers(8)
        Hp, Hm = H.copy(), H.copy()
        Hp[t, j] += h
        Hm[t, j] -= h
        assert (loss(Hp, W) - loss(Hm, W)) / (2 * h) == pytest.approx(dH[t, j], rel=1e-7, abs=1e-9)
    for _ in range(10):
        j, v = rng.integers(8), I[rng.integers(4), rng.integers(4)]  # columns on the support
        Wp, Wm = W.copy(), W.copy()
        Wp[j, v] += h
        Wm[j, v] -= h
        assert (loss(H, Wp) - loss(H, Wm)) / (2 * h) == pytest.approx(dW[j, v], rel=1e-7, abs=1e-9)
    assert np.all(dH[2] == 0)


def test_topk_reverse_zero_when_student_matches_teacher_on_support():
    # identity head (d = V, W = I): z = H.  Put A_t + c_t at the cached columns
    # of H_t (anything elsewhere): the student renormalised on the support is
    # the teacher's p^, so RKL = 0 and the mixed loss and gradient are (1 - r)
    # times the forward-KL ones.  K = 1 has a single outcome: RKL = 0 too.
    rng = np.random.default_rng(48)
    T, V, K = 5, 16, 4
    I = np.stack([rng.choice(V, K, replace=False) for _ in range(T)])
    A = rng.standard_normal((T, K)) * 1.5
    H = rng.standard_normal((T, V))
    c = rng.standard_normal(T) * 3.0
    for t in range(T):
        H[t, I[t]] = A[t] + c[t]
    W = np.eye(V)
    g = rng.standard_normal(T)
    for tau in (1.0, 1.9):
        kd, _, _ = O.topk_loss_forward(H, W, I, A, None, tau)
        dH0, dW0 = O.topk_loss_backward(H, W, I, A, None, tau, g)
        for r in (0.4, 1.0):
            got, _, _ = O.topk_loss_forward(H, W, I, A, None, tau, rev_weight=r)
            np.testing.assert_allclose(got, (1 - r) * kd, rtol=1e-12, atol=1e-13)
            dH, dW = O.topk_loss_backward(H, W, I, A, None, tau, g, rev_weight=r)
            np.testing.assert_allclose(dH, (1 - r) * dH0, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(dW, (1 - r) * dW0, rtol=1e-11, atol=1e-13)
    H1, W1, I1, A1, g1, _, _ = case(T=5, K=1, seed=49)
    kd1, _, _ = O.topk_loss_forward(H1, W1, I1, A1, None, 1.2)
    got1, _, _ = O.topk_loss_forward(H1, W1, I1, A1, None, 1.2, rev_weight=0.3)
    np.testing.assert_allclose(got1, 0.7 * kd1, rtol=1e-12)


# ---------------------------------------------------------------- full vocabulary: KL mixing, per-token tau
def full_case(T=6, d=8, dt=10, V=30, seed=30):
    rng = np.random.default_rng(seed)
    H, Ht = rng.standard_normal((T, d)), rng.standard_normal((T, dt))
    Ws = rng.standard_normal((d, V)) / np.sqrt(d)
    Wt = rng.standard_normal((dt, V)) * 1.5 / np.sqrt(dt)
    g = rng.standard_normal(T)
    taus = rng.uniform(0.6, 2.5, T)
    return H, Ws, Ht, Wt, g, taus


def torch_kl_both(H, Ws, Ht, Wt, taus):
    """KL(p || q) and KL(q || p) per row with torch's kl_div (log-space inputs)."""
    tau = torch.tensor(taus)[:, None]
    logq = torch.log_softmax(torch.tensor(H @ Ws) / tau, dim=1)
    logp = torch.log_softmax(torch.tensor(Ht @ Wt) / tau, dim=1)
    fwd = torch.nn.functional.kl_div(logq, logp, log_target=True, reduction="none").sum(1).numpy()
    rev = torch.nn.functional.kl_div(logp, logq, log_target=True, reduction="none").sum(1).numpy()
    return fwd, rev


def test_full_reverse_kl_is_torch_kl_div_swapped():
    H, Ws, Ht, Wt, g, taus = full_case(seed=31)
    got, _, _, krev = O.full_loss_forward(H, Ws, Ht, Wt, None, 1.0, tau_rows=taus, rev_weight=1.0)
    fwd, rev = torch_kl_both(H, Ws, Ht, Wt, taus)
    np.testing.assert_allclose(got, rev, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(krev, rev, rtol=1e-12, atol=1e-14)
    assert np.all(rev >= 0) and np.all(np.abs(rev - fwd) > 1e-6)  # the two directions differ here


def test_full_kl_mixing_is_the_convex_combination():
    H, Ws, Ht, Wt, g, taus = full_case(seed=32)
    fwd, rev = torch_kl_both(H, Ws, Ht, Wt, np.full(6, 1.3))
    for r in (0.0, 0.3, 0.8):
        got, lse_s, lse_t, krev = O.full_loss_forward(H, Ws, Ht, Wt, None, 1.3, rev_weight=r)
        np.testing.assert_allclose(got, (1 - r) * fwd + r * rev, rtol=1e-12, atol=1e-14)
        a, b, c = O.full_kl_forward(H, Ws, Ht, Wt, None, 1.3)
        np.testing.assert_allclose(lse_s, b, rtol=1e-14)
        np.testing.assert_allclose(lse_t, c, rtol=1e-14)


def test_full_per_token_tau_is_row_scaling():
    H, Ws, Ht, Wt, g, taus = full_case(seed=33)
    got, ls, lt, _ = O.full_loss_forward(H, Ws, Ht, Wt, None, 1.0, tau_rows=taus)
    want, ls1, lt1 = O.full_kl_forward(H / taus[:, None], Ws, Ht / taus[:, None], Wt, None, 1.0)
    np.testing.assert_allclose(got, want, rtol=1e-12)
    np.testing.assert_allclose(ls, ls1, rtol=1e-13)


def test_full_mixed_gradient_matches_torch_autograd():
    H, Ws, Ht, Wt, g, taus = full_case(T=5, seed=34)
    for r in (0.0, 0.4, 1.0):
        Hv = torch.tensor(H, requires_grad=True)
        Wv = torch.tensor(Ws, requires_grad=True)
        tau = torch.tensor(taus)[:, None]
        logq = torch.log_softmax((Hv @ Wv) / tau, dim=1)
        logp = torch.log_softmax(torch.tensor(Ht @ Wt) / tau, dim=1)
        fwd = torch.nn.functional.kl_div(logq, logp, log_target=True, reduction="none").sum(1)
        rev = torch.nn.functional.kl_div(logp, logq, log_target=True, reduction="none").sum(1)
        (((1 - r) * fwd + r * rev) * torch.tensor(g)).sum().backward()
        dH, dW = O.full_loss_backward(H, Ws, Ht, Wt, None, 1.0, g, tau_rows=taus, rev_weight=r)
        np.testing.assert_allclose(dH, Hv.grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(dW, Wv.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_full_mixed_finite_differences_and_mask():
    H, Ws, Ht, Wt, g, taus = full_case(T=4, d=6, dt=5, V=20, seed=35)
    mask = np.array([1, 1, 0, 1], dtype=np.uint8)
    kw = dict(tau_rows=taus, rev_weight=0.6)
    dH, dW = O.full_loss_backward(H, Ws, Ht, Wt, mask, 1.0, g, **kw)

    def loss(Hx, Wx):
        v = O.full_loss_forward(Hx, Wx, Ht, Wt, mask, 1.0, **kw)[0]
        return float((v * g).sum())

    h = 1e-6
    rng = np.random.default_rng(36)
    for _ in range(10):
        t, j = rng.integers(4), rng.integers(6)
        Hp, Hm = H.copy(), H.copy()
        Hp[t, j] += h
        Hm[t, j] -= h
        assert (loss(Hp, Ws) - loss(Hm, Ws)) / (2 * h) == pytest.approx(dH[t, j], rel=1e-7, abs=1e-9)
    for _ in range(10):
        j, v = rng.integers(6), rng.integers(20)
        Wp, Wm = Ws.copy(), Ws.copy()
        Wp[j, v] += h
        Wm[j, v] -= h
        assert (loss(H, Wp) - loss(H, Wm)) / (2 * h) == pytest.approx(dW[j, v], rel=1e-7, abs=1e-9)
    assert np.all(dH[2] == 0)


def test_full_options_defaults_and_equal_heads():
    H, Ws, Ht, Wt, g, _ = full_case(seed=37)
    a = O.full_loss_forward(H, Ws, Ht, Wt, None, 0.9)
    b = O.full_kl_forward(H, Ws, Ht, Wt, None, 0.9)
    for x, y in zip(a[:3], b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)
    v, _, _, kr = O.full_loss_forward(H, Ws, H, Ws, None, 0.9, rev_weight=0.5)
    assert np.all(np.abs(v) < 1e-13) and np.all(np.abs(kr) < 1e-13)
    dH, _ = O.full_loss_backward(H, Ws, H, Ws, None, 0.9, g, rev_weight=0.5)
    assert np.all(np.abs(dH) < 1e-13)
