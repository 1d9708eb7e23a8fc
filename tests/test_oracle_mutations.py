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

MUTATIONS = {
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
