"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong version (a dropped
term, a wrong sign, a missing temperature, an index off by one, a transposed
operand, an ignored mask) and runs the pins of ``test_oracle.py``: at least one
of them has to fail.  The mistakes are planted on the CPU, in the oracle only.
"""
import numpy as np
import pytest

from oracle import kd_oracle as O
from tests import test_oracle as P
from tests import test_oracle_options as Q
from tests import test_oracle_shard as S

PINS = [
    P.test_lse_constant_rows_closed_form, P.test_lse_matches_scipy, P.test_teacher_equal_logits,
    P.test_teacher_matches_torch_softmax_with_tau, P.test_golden_closed_form_v3, P.test_bruteforce_loops,
    P.test_kl_zero_when_student_equals_teacher, P.test_gibbs_lower_bound, P.test_k1_is_cross_entropy,
    P.test_shift_invariance_and_dw_rowsum, P.test_grad_matches_autograd_of_dense_reconstruction,
    P.test_grad_finite_differences, P.test_grad_closed_form_identity_head, P.test_tau_identity,
    P.test_full_vocab_matches_torch_kl_div, P.test_full_vocab_equals_topk_with_k_equal_v,
    P.test_full_vocab_grad_autograd, P.test_full_vocab_zero_when_heads_equal,
    P.test_masked_rows_are_exact_zero_and_nan_does_not_leak, P.test_all_rows_masked,
    P.test_index_gather_exact_on_integer_inputs, P.test_row_block_independence_and_slice_additivity,
    Q.test_partial_mass_with_every_entry_is_torch_kl_div, Q.test_partial_mass_scaling_identity,
    Q.test_partial_mass_matches_autograd_of_dense_reconstruction, Q.test_partial_mass_gradient_rows_sum_to_zero,
    Q.test_per_token_tau_is_row_scaling, Q.test_per_token_tau_gradient_is_row_scaled_plain_gradient,
    Q.test_ce_weight_one_is_torch_cross_entropy, Q.test_ce_mix_is_the_convex_combination,
    Q.test_ce_gradient_matches_torch_autograd, Q.test_all_options_finite_differences,
    Q.test_full_reverse_kl_is_torch_kl_div_swapped, Q.test_full_kl_mixing_is_the_convex_combination,
    Q.test_full_per_token_tau_is_row_scaling, Q.test_full_mixed_gradient_matches_torch_autograd,
    Q.test_full_mixed_finite_differences_and_mask,
    Q.test_topk_reverse_with_every_entry_is_the_full_vocab_reverse, Q.test_topk_reverse_is_torch_kl_div_on_the_support,
    Q.test_topk_mixed_gradient_matches_torch_autograd, Q.test_topk_reverse_finite_differences,
    Q.test_topk_reverse_zero_when_student_matches_teacher_on_support,
    lambda: S.test_partition_gives_the_unsharded_loss("plain", False),
    lambda: S.test_partition_gives_the_unsharded_loss("every", True),
    S.test_whole_head_as_one_shard, S.test_terms_against_scipy_and_the_dense_teacher,
    lambda: S.test_backward_partials_make_up_the_gradient("every"),
    lambda: S.test_full_partition_gives_the_unsharded_loss(True), S.test_full_shard_terms_against_scipy,
    lambda: S.test_full_backward_partials_make_up_the_gradient(0.4),
]


def _lse_no_shift(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(all="ignore"):
        return np.log(np.exp(x).sum(axis=-1))


def _teacher_no_tau(A, tau):
    a = np.asarray(A, dtype=np.float64)
    return a - O.logsumexp_rows(a)[:, None]


def _student_no_tau(Hb, W, tau):
    z = Hb @ W
    return z, z, O.logsumexp_rows(z)


def _dz_wrong_sign(s, L, I_rows, p, g_rows, tau):
    q = np.exp(s - L[:, None])
    r = np.repeat(np.arange(s.shape[0]), I_rows.shape[1])
    np.add.at(q, (r, I_rows.reshape(-1)), +p.reshape(-1))
    return q * (g_rows / tau)[:, None]


def _dz_no_g(s, L, I_rows, p, g_rows, tau):
    q = np.exp(s - L[:, None])
    r = np.repeat(np.arange(s.shape[0]), I_rows.shape[1])
    np.add.at(q, (r, I_rows.reshape(-1)), -p.reshape(-1))
    return q / tau


def _dz_no_tau(s, L, I_rows, p, g_rows, tau):
    q = np.exp(s - L[:, None])
    r = np.repeat(np.arange(s.shape[0]), I_rows.shape[1])
    np.add.at(q, (r, I_rows.reshape(-1)), -p.reshape(-1))
    return q * g_rows[:, None]


def _dz_overwrite_duplicates(s, L, I_rows, p, g_rows, tau):
    q = np.exp(s - L[:, None])
    for t in range(s.shape[0]):
        q[t, I_rows[t]] = np.exp(s[t, I_rows[t]] - L[t]) - p[t]  # duplicates overwrite
    return q * (g_rows / tau)[:, None]


def _valid_rows_ignore_mask(mask, T):
    return np.ones(T, dtype=bool)


def _make_forward_variant(kind):
    orig = O.topk_kl_forward

    def fwd(H, W, I, A, mask, tau, row_block=64):
        H, W, A = O.as_f64(H), O.as_f64(W), O.as_f64(A)
        I = np.asarray(I.cpu().numpy() if hasattr(I, "cpu") else I, dtype=np.int64)
        T, K = I.shape
        valid = O._valid_rows(mask, T)
        kl, lse, ztk = np.zeros(T), np.zeros(T), np.zeros((T, K))
        rows = np.nonzero(valid)[0]
        for r0 in range(0, rows.size, row_block):
            rb = rows[r0:r0 + row_block]
            z, s, L = O._student_block(H[rb], W, tau)
            logp = O.teacher_log_probs(A[rb], tau)
            p = np.exp(logp)
            Ib = I[rb]
            if kind == "index_off_by_one":
                Ib = (Ib + 1) % W.shape[1]
            s_at = np.take_along_axis(s, Ib, axis=1)
            if kind == "drop_entropy":
                kl[rb] = (p * (-s_at + L[:, None])).sum(axis=1)
            elif kind == "cross_sign":
                kl[rb] = (p * (logp + s_at + L[:, None])).sum(axis=1)
            elif kind == "drop_logz":
                kl[rb] = (p * (logp - s_at)).sum(axis=1)
            else:
                kl[rb] = (p * (logp - s_at + L[:, None])).sum(axis=1)
            lse[rb] = L
            ztk[rb] = np.take_along_axis(z, Ib, axis=1)
        return kl, lse, ztk

    fwd.orig = orig
    return fwd


def _backward_transposed(H, W, I, A, mask, tau, g, row_block=64, v_panel=16384):
    dH, dW = _ORIG_BWD(H, W, I, A, mask, tau, g, row_block, v_panel)
    return dH, -dW  # dW = -(H^T dZ): a sign slip in the weight gradient


_ORIG_BWD = O.topk_kl_backward


def _full_fwd_swapped(H, Ws, Ht, Wt, mask, tau, row_block=64):
    # reverse direction KL(q || p) instead of KL(p || q)
    return _ORIG_FULL(Ht, Wt, H, Ws, mask, tau, row_block)


_ORIG_FULL = O.full_kl_forward

_ORIG_LOSS_BLOCK = O._loss_block
_ORIG_LOSS_DZ = O._loss_dz
_ORIG_LOSS_FWD = O.topk_loss_forward


def _loss_block_unit_mass(H, W, A, rb, taus, tlse):
    z, s, L, p, logp, m = _ORIG_LOSS_BLOCK(H, W, A, rb, taus, tlse)
    return z, s, L, p, logp, np.ones_like(m)  # the mass term drops to 1 * log Z


def _loss_block_renormalised(H, W, A, rb, taus, tlse):
    return _ORIG_LOSS_BLOCK(H, W, A, rb, taus, None)  # teacher_lse ignored


def _row_values_ignored(x, T, default):
    return np.full(T, default, dtype=np.float64)  # tau_rows (and teacher_lse) ignored


def _loss_dz_no_onehot(s, L, I_rows, p, m, y_rows, beta, g_rows, tau_rows):
    D = _ORIG_LOSS_DZ(s, L, I_rows, p, m, y_rows, beta, g_rows, tau_rows)
    if y_rows is not None and beta != 0.0:
        D[np.arange(s.shape[0]), y_rows] += beta * g_rows / tau_rows  # the label's -1 dropped
    return D


def _loss_dz_no_mass(s, L, I_rows, p, m, y_rows, beta, g_rows, tau_rows):
    return _ORIG_LOSS_DZ(s, L, I_rows, p, np.ones_like(m), y_rows, beta, g_rows, tau_rows)


def _loss_dz_scalar_tau(s, L, I_rows, p, m, y_rows, beta, g_rows, tau_rows):
    return _ORIG_LOSS_DZ(s, L, I_rows, p, m, y_rows, beta, g_rows, np.full_like(tau_rows, tau_rows.mean()))


def _loss_fwd_weights_swapped(*args, labels=None, ce_weight=0.0, **kw):
    b = 1.0 - ce_weight if labels is not None else ce_weight
    return _ORIG_LOSS_FWD(*args, labels=labels, ce_weight=b, **kw)


def _loss_fwd_ce_sign(*args, labels=None, ce_weight=0.0, **kw):
    mix = _ORIG_LOSS_FWD(*args, labels=labels, ce_weight=ce_weight, **kw)
    if labels is None or ce_weight == 0.0:
        return mix
    kd = _ORIG_LOSS_FWD(*args, **kw)[0]
    ce = (mix[0] - (1.0 - ce_weight) * kd) / ce_weight
    return ((1.0 - ce_weight) * kd - ce_weight * ce,) + tuple(mix[1:])


_ORIG_FULL_DZ = O._full_loss_dz
_ORIG_FULL_LOSS = O.full_loss_forward


def _full_dz_no_klr(s, u, Ls, Lt, q, p, g_rows, tau_rows, r):
    D = (1.0 - r) * (q - p)
    if r != 0.0:
        D = D + r * q * ((s - Ls[:, None]) - (u - Lt[:, None]))  # the -KLr baseline dropped
    return D * (g_rows / tau_rows)[:, None]


def _full_dz_reverse_sign(s, u, Ls, Lt, q, p, g_rows, tau_rows, r):
    D = _ORIG_FULL_DZ(s, u, Ls, Lt, q, p, g_rows, tau_rows, 0.0) * (1.0 - r)
    if r != 0.0:
        D = D - _ORIG_FULL_DZ(s, u, Ls, Lt, q, p, g_rows, tau_rows, 1.0) * r
    return D


def _full_loss_mix_swapped(*args, rev_weight=0.0, **kw):
    return _ORIG_FULL_LOSS(*args, rev_weight=1.0 - rev_weight, **kw)


def _full_block_scalar_tau(H, Ws, Ht, Wt, rb, taus):
    return _ORIG_FULL_BLOCK(H, Ws, Ht, Wt, rb, np.full_like(taus, taus.mean()))


_ORIG_FULL_BLOCK = O._full_block
_ORIG_SHARD_TERMS = O.topk_shard_terms
_ORIG_SHARD_BWD = O.topk_shard_backward


def _shard_terms_unshifted(H, W_shard, v0, *args, **kw):
    return _ORIG_SHARD_TERMS(H, W_shard, 0, *args, **kw)  # global indices taken as the shard's columns


def _shard_terms_ce_ignored(*args, labels=None, ce_weight=0.0, **kw):
    return _ORIG_SHARD_TERMS(*args, **kw)


def _shard_terms_entropy_unweighted(*args, labels=None, ce_weight=0.0, **kw):
    ls, cross, ent, mass = _ORIG_SHARD_TERMS(*args, labels=labels, ce_weight=ce_weight, **kw)
    if labels is not None and ce_weight:
        ent = ent / (1.0 - ce_weight)
    return ls, cross, ent, mass


def _shard_bwd_first_columns(H, W, v0, Vs, *args, **kw):
    return _ORIG_SHARD_BWD(H, W, 0, Vs, *args, **kw)


_ORIG_FULL_SHARD_TERMS = O.full_shard_terms
_ORIG_FULL_SHARD_BWD = O.full_shard_backward


def _full_shard_heads_swapped(H, Ws_shard, Ht, Wt_shard, *args, **kw):
    ls, lt, ef, er = _ORIG_FULL_SHARD_TERMS(H, Ws_shard, Ht, Wt_shard, *args, **kw)
    return ls, lt, er, ef  # forward and reverse expectations exchanged


def _full_shard_tau_rows_ignored(*args, tau_rows=None, **kw):
    return _ORIG_FULL_SHARD_TERMS(*args, **kw)


def _full_shard_bwd_no_mixing(*args, rev_weight=0.0, **kw):
    return _ORIG_FULL_SHARD_BWD(*args, **kw)

_ORIG_SUPPORT_REV = O._support_reverse
_ORIG_LOSS_BWD = O.topk_loss_backward


def _support_rev_no_baseline(a, b):
    lq = a - O.logsumexp_rows(a)[:, None]
    lp = b - O.logsumexp_rows(b)[:, None]
    q = np.exp(lq)
    return (q * (lq - lp)).sum(axis=1), q * (lq - lp)  # the -RKL baseline dropped


def _support_rev_teacher_unnormalised(a, b):
    lq = a - O.logsumexp_rows(a)[:, None]
    q = np.exp(lq)
    rkl = (q * (lq - b)).sum(axis=1)  # A / tau taken as log p^ without renormalising
    return rkl, q * (lq - b - rkl[:, None])


def _support_rev_direction_swapped(a, b):
    return _ORIG_SUPPORT_REV(b, a)[0], _ORIG_SUPPORT_REV(a, b)[1]  # KL(p^ || q~) in the forward


def _support_rev_student_unnormalised(a, b):
    lp = b - O.logsumexp_rows(b)[:, None]
    q = np.exp(a - O.logsumexp_rows(a)[:, None])
    rkl = (q * (a - lp)).sum(axis=1)  # log q~ without its log-normaliser
    return rkl, q * (a - lp - rkl[:, None])


def _loss_fwd_rev_swapped(*args, rev_weight=0.0, **kw):
    return _ORIG_LOSS_FWD(*args, rev_weight=1.0 - rev_weight if rev_weight else 0.0, **kw)


def _loss_bwd_rev_ignores_ce(*args, labels=None, ce_weight=0.0, rev_weight=0.0, **kw):
    # the reverse part's gradient taken at full weight r, not (1 - beta) r
    dH, dW = _ORIG_LOSS_BWD(*args, labels=labels, ce_weight=ce_weight, rev_weight=rev_weight, **kw)
    if labels is None or ce_weight == 0.0 or rev_weight == 0.0:
        return dH, dW
    a = _ORIG_LOSS_BWD(*args, labels=labels, ce_weight=ce_weight, rev_weight=0.0, **kw)
    b = _ORIG_LOSS_BWD(*args, labels=labels, ce_weight=ce_weight, rev_weight=rev_weight, **kw)
    k = 1.0 / (1.0 - ce_weight)
    return tuple(None if x is None else x0 + k * (x1 - x0) for x, x0, x1 in zip((dH, dW), a, b))


MUTATIONS = {
    "topk_reverse_baseline_dropped": ("_support_reverse", _support_rev_no_baseline),
    "topk_reverse_teacher_unnormalised": ("_support_reverse", _support_rev_teacher_unnormalised),
    "topk_reverse_direction_swapped": ("_support_reverse", _support_rev_direction_swapped),
    "topk_reverse_student_unnormalised": ("_support_reverse", _support_rev_student_unnormalised),
    "topk_reverse_mix_weights_swapped": ("topk_loss_forward", _loss_fwd_rev_swapped),
    "topk_reverse_gradient_ignores_ce_weight": ("topk_loss_backward", _loss_bwd_rev_ignores_ce),
    "shard_indices_not_shifted": ("topk_shard_terms", _shard_terms_unshifted),
    "shard_ce_term_ignored": ("topk_shard_terms", _shard_terms_ce_ignored),
    "shard_entropy_unweighted": ("topk_shard_terms", _shard_terms_entropy_unweighted),
    "shard_backward_wrong_columns": ("topk_shard_backward", _shard_bwd_first_columns),
    "full_shard_expectations_swapped": ("full_shard_terms", _full_shard_heads_swapped),
    "full_shard_tau_rows_ignored": ("full_shard_terms", _full_shard_tau_rows_ignored),
    "full_shard_backward_mixing_ignored": ("full_shard_backward", _full_shard_bwd_no_mixing),
    "full_dz_reverse_baseline_dropped": ("_full_loss_dz", _full_dz_no_klr),
    "full_dz_reverse_sign": ("_full_loss_dz", _full_dz_reverse_sign),
    "full_mix_weights_swapped": ("full_loss_forward", _full_loss_mix_swapped),
    "full_tau_rows_ignored": ("_full_block", _full_block_scalar_tau),
    "loss_mass_term_unit": ("_loss_block", _loss_block_unit_mass),
    "loss_partial_mass_renormalised": ("_loss_block", _loss_block_renormalised),
    "loss_tau_rows_ignored": ("_row_values", _row_values_ignored),
    "loss_dz_label_onehot_dropped": ("_loss_dz", _loss_dz_no_onehot),
    "loss_dz_mass_dropped": ("_loss_dz", _loss_dz_no_mass),
    "loss_dz_scalar_tau": ("_loss_dz", _loss_dz_scalar_tau),
    "loss_ce_weights_swapped": ("topk_loss_forward", _loss_fwd_weights_swapped),
    "loss_ce_sign_flipped": ("topk_loss_forward", _loss_fwd_ce_sign),
    "lse_without_max_shift": ("logsumexp_rows", _lse_no_shift),
    "teacher_without_tau": ("teacher_log_probs", _teacher_no_tau),
    "student_without_tau": ("_student_block", _student_no_tau),
    "dz_wrong_sign": ("_topk_dz", _dz_wrong_sign),
    "dz_without_g": ("_topk_dz", _dz_no_g),
    "dz_without_tau": ("_topk_dz", _dz_no_tau),
    "dz_duplicates_overwrite": ("_topk_dz", _dz_overwrite_duplicates),
    "mask_ignored": ("_valid_rows", _valid_rows_ignore_mask),
    "kl_drops_teacher_entropy": ("topk_kl_forward", _make_forward_variant("drop_entropy")),
    "kl_cross_term_sign": ("topk_kl_forward", _make_forward_variant("cross_sign")),
    "kl_drops_log_z": ("topk_kl_forward", _make_forward_variant("drop_logz")),
    "gather_index_off_by_one": ("topk_kl_forward", _make_forward_variant("index_off_by_one")),
    "dw_sign_slip": ("topk_kl_backward", _backward_transposed),
    "full_kl_reversed_direction": ("full_kl_forward", _full_fwd_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # an assertion or a shape error both count as caught
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name!r}"
