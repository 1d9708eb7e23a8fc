"""Pins of the oracle's vocabulary-shard terms (``topk_shard_*``,
``full_shard_*``): the output head split by vocabulary columns across
tensor-parallel ranks ("Efficient Knowledge Distillation for LLMs: Offline
Top-K Logits and a Fused Chunked KL Loss", App. B: the loss benchmark reports
the largest tensor-parallel rank).  CPU only.

Each pin ties the shard terms to something other than their own formula: the
already pinned unsharded oracle through the partition identities (the shards'
log-normalisers log-sum-exp to L, the cross terms add, the loss comes back
from the teacher terms; the dH partials add to dH and the dW slices make up
dW), scipy's logsumexp over the shard's columns, the dense reconstruction of
the support weights (§3 "Offline implementations"), and scipy's relative
entropy of the two heads' softmaxes restricted to the shard.
"""
import numpy as np
import pytest
import scipy.special as sps

from oracle import kd_oracle as O
from tests.test_oracle_options import case, teacher_lse_for_mass

CUTS = (0, 8, 24, 40)  # three uneven shards of V = 40


def shards(V=40, cuts=CUTS):
    return [(a, b - a) for a, b in zip(cuts[:-1], cuts[1:])]


def options(name, T, taus, y, A, seed):
    rng = np.random.default_rng(seed)
    if name == "plain":
        return {}
    if name == "every":
        tl, _ = teacher_lse_for_mass(A, taus, rng)
        return dict(tau_rows=taus, teacher_lse=tl, labels=y, ce_weight=0.3)
    raise ValueError(name)


@pytest.mark.parametrize("opt", ["plain", "every"])
@pytest.mark.parametrize("dup", [False, True])
def test_partition_gives_the_unsharded_loss(opt, dup):
    H, W, I, A, g, taus, y = case(T=7, V=40, K=6, seed=11, dup=dup)
    mask = np.array([1, 1, 0, 1, 1, 1, 0], dtype=np.uint8)
    kw = options(opt, 7, taus, y, A, 12)
    tau = 1.3
    loss, L, _ = O.topk_loss_forward(H, W, I, A, mask, tau, **kw)
    parts = [O.topk_shard_terms(H, W[:, v0:v0 + vs], v0, I, A, mask, tau, **kw) for v0, vs in shards()]
    lse_s = np.stack([p[0] for p in parts])
    v = mask != 0
    np.testing.assert_allclose(sps.logsumexp(lse_s[:, v], axis=0), L[v], rtol=1e-13)
    ent, mass = parts[0][2], parts[0][3]
    for p in parts[1:]:  # the teacher terms do not depend on the shard
        np.testing.assert_array_equal(p[2], ent)
        np.testing.assert_array_equal(p[3], mass)
    cross = sum(p[1] for p in parts)
    np.testing.assert_allclose((ent - cross + mass * L)[v], loss[v], rtol=1e-12, atol=1e-13)
    for p in parts:
        for x in p:
            assert np.all(x[~v] == 0)


def test_whole_head_as_one_shard():
    H, W, I, A, g, taus, y = case(T=5, V=40, K=6, seed=13)
    loss, L, _ = O.topk_loss_forward(H, W, I, A, None, 0.8)
    ls, cross, ent, mass = O.topk_shard_terms(H, W, 0, I, A, None, 0.8)
    np.testing.assert_allclose(ls, L, rtol=1e-14)
    np.testing.assert_allclose(mass, 1.0, rtol=1e-14)
    np.testing.assert_allclose(ent - cross + L, loss, rtol=1e-12, atol=1e-13)


def test_terms_against_scipy_and_the_dense_teacher():
    # the shard's log-normaliser is scipy's logsumexp over its columns; its
    # cross term is the dense teacher weights (scatter-added support, label
    # included) dotted with s over the same columns
    H, W, I, A, g, taus, y = case(T=6, V=40, K=6, seed=14, dup=True)
    beta = 0.25
    tau = 1.1
    for v0, vs in shards():
        ls, cross, ent, mass = O.topk_shard_terms(H, W[:, v0:v0 + vs], v0, I, A, None, tau, labels=y,
                                                  ce_weight=beta)
        s = (H @ W) / tau
        np.testing.assert_allclose(ls, sps.logsumexp(s[:, v0:v0 + vs], axis=1), rtol=1e-14)
        p = sps.softmax(A / tau, axis=1)
        dense = np.zeros_like(s)
        for t in range(6):
            for k in range(6):
                dense[t, I[t, k]] += (1 - beta) * p[t, k]
            dense[t, y[t]] += beta
        np.testing.assert_allclose(cross, (dense[:, v0:v0 + vs] * s[:, v0:v0 + vs]).sum(1), rtol=1e-12,
                                   atol=1e-14)
        np.testing.assert_allclose(ent, (1 - beta) * (p * np.log(p)).sum(1), rtol=1e-13)
        np.testing.assert_allclose(mass, 1.0, rtol=1e-14)


@pytest.mark.parametrize("opt", ["plain", "every"])
def test_backward_partials_make_up_the_gradient(opt):
    H, W, I, A, g, taus, y = case(T=7, V=40, K=6, seed=15)
    mask = np.array([1, 0, 1, 1, 1, 1, 1], dtype=np.uint8)
    kw = options(opt, 7, taus, y, A, 16)
    dH, dW = O.topk_loss_backward(H, W, I, A, mask, 0.9, g, **kw)
    parts = [O.topk_shard_backward(H, W, v0, vs, I, A, mask, 0.9, g, **kw) for v0, vs in shards()]
    np.testing.assert_allclose(sum(p[0] for p in parts), dH, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate([p[1] for p in parts], axis=1), dW, rtol=1e-12, atol=1e-14)
    assert np.all(parts[1][0][1] == 0)


# ---------------------------------------------------------------- full vocabulary
def full_case(T=7, d=8, dt=6, V=40, seed=21):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((T, d))
    Ws = rng.standard_normal((d, V)) / np.sqrt(d)
    Ht = rng.standard_normal((T, dt))
    Wt = rng.standard_normal((dt, V)) * 1.5 / np.sqrt(dt)
    return H, Ws, Ht, Wt, rng.standard_normal(T), rng.uniform(0.6, 2.5, T)


@pytest.mark.parametrize("per_row_tau", [False, True])
def test_full_partition_gives_the_unsharded_loss(per_row_tau):
    H, Ws, Ht, Wt, g, taus = full_case()
    mask = np.array([1, 1, 0, 1, 1, 1, 1], dtype=np.uint8)
    tr = taus if per_row_tau else None
    v = mask != 0
    for r in (0.0, 0.35):
        loss, Ls, Lt, krev = O.full_loss_forward(H, Ws, Ht, Wt, mask, 1.1, tau_rows=tr, rev_weight=r)
        parts = [O.full_shard_terms(H, Ws[:, a:a + n], Ht, Wt[:, a:a + n], mask, 1.1, tau_rows=tr)
                 for a, n in shards()]
        ls, lt, ef, er = (np.stack([p[i] for p in parts]) for i in range(4))
        np.testing.assert_allclose(sps.logsumexp(ls[:, v], axis=0), Ls[v], rtol=1e-13)
        np.testing.assert_allclose(sps.logsumexp(lt[:, v], axis=0), Lt[v], rtol=1e-13)
        fwd = (np.exp(lt - Lt) * ef).sum(0) - Lt + Ls
        rev = (np.exp(ls - Ls) * er).sum(0) - Ls + Lt
        np.testing.assert_allclose(((1 - r) * fwd + r * rev)[v], loss[v], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(rev[v], krev[v], rtol=1e-11, atol=1e-13)
        for p in parts:
            for x in p:
                assert np.all(x[~v] == 0)


def test_full_shard_terms_against_scipy():
    # each shard's terms are the KL pieces of the two softmaxes restricted to its columns
    H, Ws, Ht, Wt, g, taus = full_case(seed=22)
    for a, n in shards():
        ls, lt, ef, er = O.full_shard_terms(H, Ws[:, a:a + n], Ht, Wt[:, a:a + n], None, 0.8)
        s, u = (H @ Ws[:, a:a + n]) / 0.8, (Ht @ Wt[:, a:a + n]) / 0.8
        np.testing.assert_allclose(ls, sps.logsumexp(s, axis=1), rtol=1e-14)
        np.testing.assert_allclose(lt, sps.logsumexp(u, axis=1), rtol=1e-14)
        P, Q = sps.softmax(u, axis=1), sps.softmax(s, axis=1)
        # sum P (u - s) = KL(P || Q) + lse_t - lse_s over the shard's columns, likewise e_rev
        np.testing.assert_allclose(ef, sps.rel_entr(P, Q).sum(1) + lt - ls, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(er, sps.rel_entr(Q, P).sum(1) + ls - lt, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("r", [0.0, 0.4])
def test_full_backward_partials_make_up_the_gradient(r):
    H, Ws, Ht, Wt, g, taus = full_case(seed=23)
    mask = np.array([1, 1, 1, 0, 1, 1, 1], dtype=np.uint8)
    dH, dW = O.full_loss_backward(H, Ws, Ht, Wt, mask, 1.2, g, tau_rows=taus, rev_weight=r)
    parts = [O.full_shard_backward(H, Ws, Ht, Wt, a, n, mask, 1.2, g, tau_rows=taus, rev_weight=r)
             for a, n in shards()]
    np.testing.assert_allclose(sum(p[0] for p in parts), dH, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate([p[1] for p in parts], axis=1), dW, rtol=1e-12, atol=1e-14)
    assert np.all(parts[0][0][3] == 0)
