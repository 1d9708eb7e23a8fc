"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
closed forms, library routines, finite differences, brute-force loops and a
hand-derived worked example.  CPU only.

The loss is the forward KL of "Efficient Knowledge Distillation for LLMs:
Offline Top-K Logits and a Fused Chunked KL Loss" (§1, §3 "Offline
distillation": support-entry terms plus one full-vocabulary log Z) and, for the
full-vocabulary variant, the frozen-teacher-head recompute of the KDFlow
abstract.  Each pin says which mistake it would catch.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

from oracle import kd_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(T=6, d=8, V=32, K=4, seed=0, tau=1.0, dup=False):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, d))
    W = rng.standard_normal((d, V)) / np.sqrt(d)
    A = -np.sort(-rng.standard_normal((T, K)) * 1.7, axis=1)
    I = np.stack([rng.choice(V, K, replace=False) for _ in range(T)]).astype(np.int64)
    if dup:
        I[:, 1] = I[:, 0]
    g = rng.standard_normal(T)
    return H, W, I, A, g, tau


# ---------------------------------------------------------------- P1: log Z
def test_lse_constant_rows_closed_form():
    # constant logits c over V entries: log Z = c + log V
    for c, V in [(0.0, 7), (3.5, 4096), (-1200.0, 100), (800.0, 3)]:
        x = np.full((2, V), c)
        np.testing.assert_allclose(O.logsumexp_rows(x), c + math.log(V), rtol=1e-15, atol=1e-12)


def test_lse_matches_scipy():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 1000)) * 30
    np.testing.assert_allclose(O.logsumexp_rows(x), sps.logsumexp(x, axis=1), rtol=1e-14)


# ---------------------------------------------------------------- P2: teacher
def test_teacher_equal_logits():
    # equal teacher logits: p = 1/K and sum p log p = -log K
    for K in (1, 2, 16, 64):
        lp = O.teacher_log_probs(np.full((3, K), 0.37), tau=1.7)
        np.testing.assert_allclose(np.exp(lp), 1.0 / K, rtol=1e-14)
        np.testing.assert_allclose((np.exp(lp) * lp).sum(1), -math.log(K), rtol=1e-14, atol=1e-15)


def test_teacher_matches_torch_softmax_with_tau():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((4, 9)) * 3
    for tau in (0.5, 1.0, 2.0):
        ref = torch.log_softmax(torch.tensor(A, dtype=torch.float64) / tau, dim=1).numpy()
        np.testing.assert_allclose(O.teacher_log_probs(A, tau), ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- golden: worked example
def test_golden_closed_form_v3():
    with open(os.path.join(GOLDEN, "closed_form_v3.json")) as f:
        G = json.load(f)
    s = np.array([[0.0, math.log(2), math.log(3)]])
    I = np.array([G["topk_idx"]])
    A = np.array([[math.log(3), 0.0]])
    W = np.eye(3)
    kl, lse, ztk = O.topk_kl_forward(s, W, I, A, None, 1.0)
    assert kl[0] == pytest.approx(G["kl"], rel=1e-14)
    assert kl[0] == pytest.approx(0.75 * math.log(1.5) + 0.25 * math.log(0.75), rel=1e-14)
    assert lse[0] == pytest.approx(G["lse"], rel=1e-15)
    np.testing.assert_allclose(ztk[0], [math.log(3), math.log(2)], rtol=1e-15)
    # W = identity makes dH = dZ: the closed-form gradient q - scatter(p)
    dH, dW = O.topk_kl_backward(s, W, I, A, None, 1.0, np.ones(1))
    np.testing.assert_allclose(dH[0], G["dz"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dW, np.outer(s[0], G["dz"]), rtol=1e-13, atol=1e-15)
    # tau = 2: same closed form with halved logits
    q = np.exp(s[0] / 2); q /= q.sum()
    p = np.exp(A[0] / 2); p /= p.sum()
    want = p[0] * math.log(p[0] / q[2]) + p[1] * math.log(p[1] / q[1])
    kl2, _, _ = O.topk_kl_forward(s, W, I, A, None, 2.0)
    assert kl2[0] == pytest.approx(want, rel=1e-13)


# ---------------------------------------------------------------- brute force
def _brute_topk_kl(H, W, I, A, tau):
    """Scalar-loop definition with math.exp/log only (tiny inputs)."""
    T, d = len(H), len(H[0])
    V, K = len(W[0]), len(I[0])
    out = []
    for t in range(T):
        s = [sum(H[t][j] * W[j][v] for j in range(d)) / tau for v in range(V)]
        zmax = max(s)
        logZ = zmax + math.log(sum(math.exp(x - zmax) for x in s))
        a = [A[t][k] / tau for k in range(K)]
        amax = max(a)
        logZa = amax + math.log(sum(math.exp(x - amax) for x in a))
        kl = 0.0
        for k in range(K):
            lp = a[k] - logZa
            lq = s[I[t][k]] - logZ
            kl += math.exp(lp) * (lp - lq)
        out.append(kl)
    return out


def test_bruteforce_loops():
    for tau in (1.0, 0.7, 2.0):
        H, W, I, A, g, _ = rand_case(T=3, d=4, V=7, K=3, seed=3)
        want = _brute_topk_kl(H.tolist(), W.tolist(), I.tolist(), A.tolist(), tau)
        kl, _, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        np.testing.assert_allclose(kl, want, rtol=1e-12)


# ---------------------------------------------------------------- P3: KL = 0
def test_kl_zero_when_student_equals_teacher():
    # K = V, I_t a permutation, W = identity and H_t[I_tk] = A_tk: s_I = a, so KL = 0
    rng = np.random.default_rng(4)
    V = 16
    T = 5
    A = -np.sort(-rng.standard_normal((T, V)), axis=1)
    I = np.stack([rng.permutation(V) for _ in range(T)])
    H = np.zeros((T, V))
    for t in range(T):
        H[t, I[t]] = A[t]
    for tau in (1.0, 3.0):
        kl, _, _ = O.topk_kl_forward(H, np.eye(V), I, A, None, tau)
        np.testing.assert_allclose(kl, 0.0, atol=1e-14)
        dH, dW = O.topk_kl_backward(H, np.eye(V), I, A, None, tau, np.ones(T))
        np.testing.assert_allclose(dH, 0.0, atol=1e-15)
        np.testing.assert_allclose(dW, 0.0, atol=1e-14)


# ---------------------------------------------------------------- P4: Gibbs
def test_gibbs_lower_bound():
    for seed in range(5):
        H, W, I, A, g, tau = rand_case(T=20, d=8, V=50, K=6, seed=seed)
        kl, lse, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        s = H @ W
        q = np.exp(s - sps.logsumexp(s, axis=1, keepdims=True))
        bound = -np.log(np.take_along_axis(q, I, axis=1).sum(1))
        assert np.all(kl >= bound - 1e-12)
        assert np.all(bound >= 0)


# ---------------------------------------------------------------- P5: K = 1 is cross-entropy
def test_k1_is_cross_entropy():
    H, W, I, A, g, tau = rand_case(T=9, d=8, V=40, K=1, seed=5)
    for tau in (1.0, 1.5):
        kl, _, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        logits = torch.tensor(H @ W / tau)
        ce = torch.nn.functional.cross_entropy(logits, torch.tensor(I[:, 0]), reduction="none").numpy()
        np.testing.assert_allclose(kl, ce, rtol=1e-13)


# ---------------------------------------------------------------- P6: shift invariance
def test_shift_invariance_and_dw_rowsum():
    H, W, I, A, g, tau = rand_case(T=7, d=8, V=30, K=5, seed=6)
    u = np.random.default_rng(7).standard_normal(8)
    W2 = W + u[:, None]  # every logit of row t moves by H_t . u
    kl1, _, _ = O.topk_kl_forward(H, W, I, A, None, tau)
    kl2, _, _ = O.topk_kl_forward(H, W2, I, A, None, tau)
    np.testing.assert_allclose(kl1, kl2, rtol=1e-12)
    dH1, dW1 = O.topk_kl_backward(H, W, I, A, None, tau, g)
    dH2, _ = O.topk_kl_backward(H, W2, I, A, None, tau, g)
    np.testing.assert_allclose(dH1, dH2, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dW1.sum(1), 0.0, atol=1e-13)  # sum_v dZ = 0 with mass 1


# ---------------------------------------------------------------- P7: gradients
def _dense_reconstruction_loss(Ht, Wt, I, A, mask, tau, g):
    """The dense variant of [EKD] §3: scatter the teacher top-K into a dense
    [T, V] distribution and take KL against the full student log-softmax."""
    T, V = Ht.shape[0], Wt.shape[1]
    logq = torch.log_softmax((Ht @ Wt) / tau, dim=1)
    p = torch.softmax(torch.tensor(A, dtype=torch.float64) / tau, dim=1)
    P = torch.zeros(T, V, dtype=torch.float64)
    P.scatter_add_(1, torch.tensor(I), p)
    plogp = torch.where(P > 0, P * torch.log(torch.where(P > 0, P, torch.ones_like(P))), torch.zeros_like(P))
    kl = (plogp - P * logq).sum(1)
    m = torch.ones(T, dtype=torch.float64) if mask is None else torch.tensor(mask, dtype=torch.float64)
    return (kl * m * torch.tensor(g)).sum(), kl


def test_grad_matches_autograd_of_dense_reconstruction():
    for tau, dup in [(1.0, False), (0.8, False), (2.0, True)]:
        H, W, I, A, g, _ = rand_case(T=8, d=6, V=25, K=5, seed=8, dup=dup)
        mask = np.array([1, 1, 0, 1, 1, 1, 0, 1], dtype=np.uint8)
        Ht = torch.tensor(H, requires_grad=True)
        Wt = torch.tensor(W, requires_grad=True)
        loss, kl_dense = _dense_reconstruction_loss(Ht, Wt, I, A, mask, tau, g)
        loss.backward()
        kl, _, _ = O.topk_kl_forward(H, W, I, A, mask, tau)
        # duplicate indices merge their mass in the dense tensor; the sparse identity
        # keeps them apart, so the forward values differ there (the gradients agree)
        if not dup:
            np.testing.assert_allclose(kl[mask == 1], kl_dense.detach().numpy()[mask == 1], rtol=1e-12)
        dH, dW = O.topk_kl_backward(H, W, I, A, mask, tau, g)
        np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_grad_finite_differences():
    H, W, I, A, g, tau = rand_case(T=4, d=8, V=32, K=4, seed=9, tau=1.3)
    dH, dW = O.topk_kl_backward(H, W, I, A, None, tau, g)

    def loss(Hx, Wx):
        kl, _, _ = O.topk_kl_forward(Hx, Wx, I, A, None, tau)
        return float((kl * g).sum())

    h = 1e-6
    rng = np.random.default_rng(10)
    for _ in range(12):
        t, j = rng.integers(4), rng.integers(8)
        Hp, Hm = H.copy(), H.copy()
        Hp[t, j] += h
        Hm[t, j] -= h
        fd = (loss(Hp, W) - loss(Hm, W)) / (2 * h)
        assert fd == pytest.approx(dH[t, j], rel=1e-7, abs=1e-9)
    for _ in range(12):
        j, v = rng.integers(8), rng.integers(32)
        Wp, Wm = W.copy(), W.copy()
        Wp[j, v] += h
        Wm[j, v] -= h
        fd = (loss(H, Wp) - loss(H, Wm)) / (2 * h)
        assert fd == pytest.approx(dW[j, v], rel=1e-7, abs=1e-9)


def test_grad_closed_form_identity_head():
    # W = I: dH = dZ = softmax(z) - scatter(p) at tau = 1, g = 1
    rng = np.random.default_rng(11)
    V, K, T = 20, 4, 6
    H = rng.standard_normal((T, V))
    A = rng.standard_normal((T, K))
    I = np.stack([rng.choice(V, K, replace=False) for _ in range(T)])
    dH, _ = O.topk_kl_backward(H, np.eye(V), I, A, None, 1.0, np.ones(T))
    want = sps.softmax(H, axis=1)
    p = sps.softmax(A, axis=1)
    for t in range(T):
        want[t, I[t]] -= p[t]
    np.testing.assert_allclose(dH, want, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- P8: temperature identity
def test_tau_identity():
    H, W, I, A, g, _ = rand_case(T=5, d=8, V=40, K=6, seed=12)
    for tau in (0.5, 2.0, 3.7):
        a, _, _ = O.topk_kl_forward(H, W, I, A, None, tau)
        b, _, _ = O.topk_kl_forward(H / tau, W, I, A / tau, None, 1.0)
        np.testing.assert_allclose(a, b, rtol=1e-12)


# ---------------------------------------------------------------- P9: full vocabulary
def test_full_vocab_matches_torch_kl_div():
    rng = np.random.default_rng(13)
    T, d, dt, V = 6, 8, 10, 30
    H, Ht = rng.standard_normal((T, d)), rng.standard_normal((T, dt))
    Ws, Wt = rng.standard_normal((d, V)) / 3, rng.standard_normal((dt, V)) / 3
    for tau in (1.0, 2.0):
        kl, ls, lt = O.full_kl_forward(H, Ws, Ht, Wt, None, tau)
        s = torch.log_softmax(torch.tensor(H @ Ws / tau), 1)
        u = torch.log_softmax(torch.tensor(Ht @ Wt / tau), 1)
        ref = torch.nn.functional.kl_div(s, u, reduction="none", log_target=True).sum(1).numpy()
        np.testing.assert_allclose(kl, ref, rtol=1e-12)
        np.testing.assert_allclose(ls, sps.logsumexp(H @ Ws / tau, axis=1), rtol=1e-14)
        np.testing.assert_allclose(lt, sps.logsumexp(Ht @ Wt / tau, axis=1), rtol=1e-14)


def test_full_vocab_equals_topk_with_k_equal_v():
    rng = np.random.default_rng(14)
    T, d, dt, V = 5, 8, 6, 24
    H, Ht = rng.standard_normal((T, d)), rng.standard_normal((T, dt))
    Ws, Wt = rng.standard_normal((d, V)) / 3, rng.standard_normal((dt, V)) / 3
    g = rng.standard_normal(T)
    I = np.tile(np.arange(V), (T, 1))
    for tau in (1.0, 1.6):
        kf, _, _ = O.full_kl_forward(H, Ws, Ht, Wt, None, tau)
        kt, _, _ = O.topk_kl_forward(H, Ws, I, Ht @ Wt, None, tau)
        np.testing.assert_allclose(kf, kt, rtol=1e-12)
        dHf, dWf = O.full_kl_backward(H, Ws, Ht, Wt, None, tau, g)
        dHt, dWt = O.topk_kl_backward(H, Ws, I, Ht @ Wt, None, tau, g)
        np.testing.assert_allclose(dHf, dHt, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(dWf, dWt, rtol=1e-11, atol=1e-14)


def test_full_vocab_grad_autograd():
    rng = np.random.default_rng(15)
    T, d, dt, V = 5, 7, 9, 21
    H, Ht = rng.standard_normal((T, d)), rng.standard_normal((T, dt))
    Ws, Wt = rng.standard_normal((d, V)) / 3, rng.standard_normal((dt, V)) / 3
    g = rng.standard_normal(T)
    mask = np.array([1, 0, 1, 1, 1], dtype=np.uint8)
    tau = 1.4
    Hx, Wx = torch.tensor(H, requires_grad=True), torch.tensor(Ws, requires_grad=True)
    s = torch.log_softmax(Hx @ Wx / tau, 1)
    u = torch.log_softmax(torch.tensor(Ht @ Wt / tau), 1)
    kl = torch.nn.functional.kl_div(s, u, reduction="none", log_target=True).sum(1)
    (kl * torch.tensor(g) * torch.tensor(mask, dtype=torch.float64)).sum().backward()
    dH, dW = O.full_kl_backward(H, Ws, Ht, Wt, mask, tau, g)
    np.testing.assert_allclose(dH, Hx.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, Wx.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_full_vocab_zero_when_heads_equal():
    rng = np.random.default_rng(16)
    H = rng.standard_normal((4, 8))
    W = rng.standard_normal((8, 40)) / 3
    kl, _, _ = O.full_kl_forward(H, W, H, W, None, 1.3)
    np.testing.assert_allclose(kl, 0.0, atol=1e-14)


# ---------------------------------------------------------------- P10: masks
def test_masked_rows_are_exact_zero_and_nan_does_not_leak():
    H, W, I, A, g, tau = rand_case(T=6, d=8, V=30, K=4, seed=17)
    mask = np.array([1, 0, 1, 0, 1, 1], dtype=np.uint8)
    Hn, An, In = H.copy(), A.copy(), I.copy()
    Hn[mask == 0] = np.nan
    An[mask == 0] = np.nan
    In[mask == 0] = 10**6  # out of range, must never be read
    kl, lse, ztk = O.topk_kl_forward(Hn, W, In, An, mask, tau)
    dH, dW = O.topk_kl_backward(Hn, W, In, An, mask, tau, g)
    assert np.all(kl[mask == 0] == 0) and np.all(lse[mask == 0] == 0) and np.all(ztk[mask == 0] == 0)
    assert np.all(dH[mask == 0] == 0)
    assert np.all(np.isfinite(dW)) and np.all(np.isfinite(kl)) and np.all(np.isfinite(dH))
    # valid rows equal the result over the valid rows alone
    v = mask == 1
    kl2, _, _ = O.topk_kl_forward(H[v], W, I[v], A[v], None, tau)
    dH2, dW2 = O.topk_kl_backward(H[v], W, I[v], A[v], None, tau, g[v])
    np.testing.assert_array_equal(kl[v], kl2)
    np.testing.assert_allclose(dH[v], dH2, rtol=1e-14)
    np.testing.assert_allclose(dW, dW2, rtol=1e-13, atol=1e-16)


def test_all_rows_masked():
    H, W, I, A, g, tau = rand_case(T=3, d=8, V=30, K=4, seed=18)
    mask = np.zeros(3, dtype=np.uint8)
    kl, lse, _ = O.topk_kl_forward(H, W, I, A, mask, tau)
    dH, dW = O.topk_kl_backward(H, W, I, A, mask, tau, g)
    assert not kl.any() and not lse.any() and not dH.any() and not dW.any()


# ---------------------------------------------------------------- P11: exact gather
def test_index_gather_exact_on_integer_inputs():
    rng = np.random.default_rng(19)
    T, d, V, K = 8, 16, 64, 8
    H = rng.integers(-2, 3, (T, d)).astype(np.float64)
    W = rng.integers(-2, 3, (d, V)).astype(np.float64) / 8
    I = np.stack([rng.choice(V, K, replace=False) for _ in range(T)])
    A = rng.standard_normal((T, K))
    _, _, ztk = O.topk_kl_forward(H, W, I, A, None, 1.0)
    Hi = H.astype(np.int64).tolist()
    W8 = (W * 8).astype(np.int64).tolist()
    for t in range(T):
        for k in range(K):
            exact = sum(Hi[t][j] * W8[j][I[t, k]] for j in range(d)) / 8
            assert ztk[t, k] == exact


# ---------------------------------------------------------------- P12: structure
def test_row_block_independence_and_slice_additivity():
    H, W, I, A, g, tau = rand_case(T=40, d=8, V=60, K=5, seed=20)
    kl_a, _, _ = O.topk_kl_forward(H, W, I, A, None, tau, row_block=7)
    kl_b, _, _ = O.topk_kl_forward(H, W, I, A, None, tau, row_block=64)
    np.testing.assert_allclose(kl_a, kl_b, rtol=1e-14)
    dH, dW = O.topk_kl_backward(H, W, I, A, None, tau, g, row_block=16, v_panel=7)
    dHa, dWa = O.topk_kl_backward(H[:17], W, I[:17], A[:17], None, tau, g[:17])
    dHb, dWb = O.topk_kl_backward(H[17:], W, I[17:], A[17:], None, tau, g[17:])
    np.testing.assert_allclose(dW, dWa + dWb, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dH, np.vstack([dHa, dHb]), rtol=1e-14)


def test_rows_helpers_match_full_functions():
    H, W, I, A, g, tau = rand_case(T=12, d=8, V=40, K=5, seed=21, tau=1.5)
    mask = np.ones(12, dtype=np.uint8)
    mask[[3, 7]] = 0
    rows = np.array([0, 3, 5, 11])
    kl, lse, ztk = O.topk_kl_forward(H, W, I, A, mask, tau)
    dH, _ = O.topk_kl_backward(H, W, I, A, mask, tau, g)
    kr, lr, zr, dHr = O.topk_kl_rows(H, W, I, A, mask, tau, g, rows)
    np.testing.assert_allclose(kr, kl[rows], rtol=1e-14)
    np.testing.assert_allclose(lr, lse[rows], rtol=1e-14)
    np.testing.assert_allclose(zr, ztk[rows], rtol=1e-14)
    np.testing.assert_allclose(dHr, dH[rows], rtol=1e-13, atol=1e-16)
    rng = np.random.default_rng(22)
    Ht = rng.standard_normal((12, 6))
    Wt = rng.standard_normal((6, 40)) / 3
    kf, lsf, ltf = O.full_kl_forward(H, W, Ht, Wt, mask, tau)
    dHf, _ = O.full_kl_backward(H, W, Ht, Wt, mask, tau, g)
    a, b, c, e = O.full_kl_rows(H, W, Ht, Wt, mask, tau, g, rows)
    np.testing.assert_allclose(a, kf[rows], rtol=1e-14)
    np.testing.assert_allclose(e, dHf[rows], rtol=1e-13, atol=1e-16)


def test_torch_inputs_bf16_are_read_exactly():
    x = torch.tensor([[1.0, 2.0 ** -9 + 1.0, -3.25]], dtype=torch.bfloat16)
    y = O.as_f64(x)
    assert y.dtype == np.float64
    assert y.tolist() == [[1.0, 1.0, -3.25]]  # 1 + 2^-9 rounds to 1 in bf16 (RNE)
