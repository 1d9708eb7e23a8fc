"""Pins of the oracle's vocabulary-shard terms (``topk_shard_terms``,
``topk_shard_backward``): the output head split by vocabulary columns across
tensor-parallel ranks ("Efficient Knowledge Distillation for LLMs: Offline
Top-K Logits and a Fused Chunked KL Loss", App. B: the loss benchmark reports
the largest tensor-parallel rank).  CPU only.

Each pin ties the shard terms to something other than their own formula: the
already pinned unsharded oracle through the partition identities (the shards'
log-normalisers log-sum-exp to L, the cross terms add, the loss comes back
from the teacher terms; the dH partials add to dH and the dW slices make up
dW), scipy's logsumexp over the shard's columns, and the dense
reconstruction of the support weights (§3 "Offline implementations").
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
