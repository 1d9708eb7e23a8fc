"""GPU parity over a seeded sweep of shapes: the HIP path against the fp64
oracle on configurations drawn once from a fixed seed, so that the kernel
selections (direct-load ring or register-staged loop), partial vocabulary and
row tiles, backward chunk counts, K, temperatures, masks and (in a stream of
its own) KL mixing with the other options are exercised in combinations the
hand-picked cases do not list.  Every case is small enough for the oracle to
finish in about a second.
"""
import numpy as np
import pytest
import torch

import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, run_full, run_topk, say

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261204)


def _draw_topk(n):
    out = []
    for i in range(n):
        dtype = torch.bfloat16 if i % 4 else torch.float32
        # bf16 widths that take the direct-load ring (multiples of 128) and
        # ones that do not
        d = int(_rng.choice([128, 256, 384, 96, 200] if dtype == torch.bfloat16 else [64, 96, 128]))
        V = int(8 * _rng.integers(33, 520))  # 264 .. 4152, a multiple of 8
        T = int(_rng.integers(1, 600))
        K = int(min(V, _rng.integers(1, 80)))
        tau = float(np.round(_rng.uniform(0.5, 2.0), 3))
        mask = str(_rng.choice(["none", "random10"]))
        chunk = int(_rng.choice([0, 64, 256, 448]))
        one_call = bool(_rng.integers(0, 2))
        out.append((i, dtype, T, d, V, K, tau, mask, chunk, one_call))
    return out


def _draw_full(n):
    out = []
    for i in range(n):
        dtype = torch.bfloat16 if i % 3 else torch.float32
        d = int(_rng.choice([128, 256, 96]))
        dt = int(_rng.choice([128, 384, 160]))
        V = int(8 * _rng.integers(33, 400))
        T = int(_rng.integers(1, 500))
        tau = float(np.round(_rng.uniform(0.5, 2.0), 3))
        mask = str(_rng.choice(["none", "random10"]))
        chunk = int(_rng.choice([0, 128, 320]))
        out.append((i, dtype, T, d, dt, V, tau, mask, chunk))
    return out


TOPK_CASES = _draw_topk(20)
FULL_CASES = _draw_full(10)

_rng_rev = np.random.default_rng(20261205)  # its own stream: the cases above stay as they were


def _draw_rev(n):
    """Top-K cases with KL mixing (rev_weight) and a random subset of the
    other options; half of them through the single call."""
    out = []
    for i in range(n):
        dtype = torch.bfloat16 if i % 3 else torch.float32
        d = int(_rng_rev.choice([128, 256, 96, 200] if dtype == torch.bfloat16 else [64, 96]))
        V = int(8 * _rng_rev.integers(33, 400))
        T = int(_rng_rev.integers(1, 500))
        K = int(min(V, _rng_rev.integers(1, 90)))
        tau = float(np.round(_rng_rev.uniform(0.5, 2.0), 3))
        r = float(np.round(_rng_rev.uniform(0.05, 1.0), 3))
        opts = dict(tau_rows=bool(_rng_rev.integers(0, 2)), partial_mass=bool(_rng_rev.integers(0, 2)))
        if _rng_rev.integers(0, 2):
            opts.update(labels=True, ce_weight=float(np.round(_rng_rev.uniform(0.1, 0.9), 3)))
        mask = str(_rng_rev.choice(["none", "random10"]))
        chunk = int(_rng_rev.choice([0, 64, 256]))
        one_call = bool(_rng_rev.integers(0, 2))
        out.append((i, dtype, T, d, V, K, tau, r, opts, mask, chunk, one_call))
    return out


REV_CASES = _draw_rev(10)


def _valid(inp):
    T = inp["H"].shape[0]
    return np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0


@pytest.mark.parametrize("case", TOPK_CASES, ids=[f"topk{c[0]}" for c in TOPK_CASES])
def test_topk_sweep(case):
    i, dtype, T, d, V, K, tau, mask, chunk, one_call = case
    inp = G.make_topk(T, d, V, K, dtype, tau=tau, mask=mask, number=300 + i, g="normal")
    say(f"sweep top-K #{i} T={T} d={d} V={V} K={K} tau={tau} mask={mask} chunk={chunk} one_call={one_call} {dtype}")
    if one_call:
        import chunked_kl_loss_logit_amd as kd
        dev = lambda x: None if x is None else x.cuda().contiguous()  # noqa: E731
        kl, lse, _, dH, dW = kd.topk_kl_forward_backward(dev(inp["H"]), dev(inp["W"]), dev(inp["I"]),
                                                         dev(inp["A"]), dev(inp["mask"]), tau, dev(inp["g"]),
                                                         chunk_rows=chunk)
        torch.cuda.synchronize()
        got = dict(kl=kl.cpu().double().numpy(), lse=lse.cpu().double().numpy(),
                   dH=dH.cpu().double().numpy(), dW=dW.cpu().double().numpy())
    else:
        got = run_topk(inp, want_z=False, chunk_rows=chunk)
    kl, lse, _ = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], tau)
    dH, dW = O.topk_kl_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], tau, inp["g"])
    v = _valid(inp)
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse"], lse, dtype, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dW")


@pytest.mark.parametrize("case", FULL_CASES, ids=[f"full{c[0]}" for c in FULL_CASES])
def test_full_sweep(case):
    i, dtype, T, d, dt, V, tau, mask, chunk = case
    inp = G.make_full(T, d, dt, V, dtype, tau=tau, mask=mask, number=400 + i, g="normal")
    say(f"sweep full #{i} T={T} d={d} dt={dt} V={V} tau={tau} mask={mask} chunk={chunk} {dtype}")
    got = run_full(inp, chunk_rows=chunk)
    kl, ls, lt = O.full_kl_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], tau)
    dH, dW = O.full_kl_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], tau, inp["g"])
    v = _valid(inp)
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse_s"], ls, dtype, v)
    assert_lse(got["lse_t"], lt, dtype, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dWs")


@pytest.mark.parametrize("case", REV_CASES, ids=[f"rev{c[0]}" for c in REV_CASES])
def test_topk_reverse_sweep(case):
    import chunked_kl_loss_logit_amd as kd
    i, dtype, T, d, V, K, tau, r, opts, mask, chunk, one_call = case
    inp = G.make_topk(T, d, V, K, dtype, tau=tau, mask=mask, number=500 + i, g="normal")
    inp = G.add_topk_options(inp, number=500 + i, **opts)
    if K > 1 and T > 3:
        I = inp["I"].clone()
        I[::3, 1] = I[::3, 0]  # repeated indices in every third row
        inp["I"] = I
    say(f"sweep reverse #{i} T={T} d={d} V={V} K={K} tau={tau} r={r} {opts} mask={mask} chunk={chunk} "
        f"one_call={one_call} {dtype}")
    dev = lambda x: None if x is None else x.cuda().contiguous()  # noqa: E731
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    o = {k: dev(inp[k]) for k in ("tau_rows", "teacher_lse", "labels") if k in inp}
    if "labels" in inp:
        o["ce_weight"] = inp["ce_weight"]
    if one_call:
        kl, lse, _, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, M, tau, g, chunk_rows=chunk, rev_weight=r, **o)
    else:
        kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, rev_weight=r, **o)
        dH, dW = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, chunk, rev_weight=r, z_topk=z, **o)
    torch.cuda.synchronize()
    kw = {k: inp[k] for k in ("tau_rows", "teacher_lse", "labels") if k in inp}
    if "labels" in inp:
        kw["ce_weight"] = inp["ce_weight"]
    want_kl, want_lse, _ = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], tau,
                                               rev_weight=r, **kw)
    wdH, wdW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], tau, inp["g"],
                                    rev_weight=r, **kw)
    v = _valid(inp)
    got_kl = kl.cpu().double().numpy()
    assert_kl(got_kl, want_kl, dtype, v)
    assert_lse(lse.cpu().double().numpy(), want_lse, dtype, v)
    assert np.all(got_kl[~v] == 0) and np.all(dH.cpu().double().numpy()[~v] == 0)
    assert_grad(dH.cpu().double().numpy(), wdH, dtype, "dH")
    assert_grad(dW.cpu().double().numpy(), wdW, dtype, "dW")
