"""GPU parity of KL mixing on the top-K loss (kd_topk_opts.rev_weight): the
reverse KL between the student and the teacher, both restricted to the K
cached entries and renormalised there, mixed with the forward KL, against the
fp64 oracle's topk_loss_* (KL-direction abstract: forward and reverse
token-level KL and their mixture; the restriction to the cached entries is the
library's reading, since the teacher is known only there).

The forward adds r RKL to each row from z_topk; the backward gets the
forward's z_topk and folds the reverse gradient into the support weights that
the dZ tiles scatter, so the tiles are the plain call's."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, say

pytestmark = pytest.mark.gpu

OPTS = ("tau_rows", "teacher_lse", "labels")


def run_rev(inp, r, chunk_rows=0, one_call=False):
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    o = {k: dev(inp[k]) for k in OPTS if k in inp}
    if "labels" in inp:
        o["ce_weight"] = inp["ce_weight"]
    tau = inp["tau"]
    if one_call:
        kl, lse, z, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, M, tau, g, chunk_rows, rev_weight=r, **o)
    else:
        kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, rev_weight=r, **o)
        dH, dW = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, chunk_rows, rev_weight=r, z_topk=z, **o)
    torch.cuda.synchronize()
    out = dict(kl=kl, lse=lse, z=z, dH=dH, dW=dW)
    return {k: v.cpu().double().numpy() for k, v in out.items() if v is not None}  # z: None at r = 0


def oracle_kw(inp, r):
    kw = {k: inp[k] for k in OPTS if k in inp}
    if "labels" in inp:
        kw["ce_weight"] = inp["ce_weight"]
    kw["rev_weight"] = r
    return kw


def check(got, inp, r, dtype):
    kw = oracle_kw(inp, r)
    kl, lse, z = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], **kw)
    dH, dW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], **kw)
    T = kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse"], lse, dtype, v)
    for k in ("kl", "lse", "dH"):
        assert np.all(got[k][~v] == 0), k
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dW")


def with_duplicates(inp, every=7):
    """Every `every`-th row repeats its first cached index in entry 1."""
    I = inp["I"].clone()
    I[::every, 1] = I[::every, 0]
    return dict(inp, I=I)


SHAPES = [
    (torch.bfloat16, 700, 384, 2568, 24, 256, "random10"),   # direct-load, shifted last tile, 3 chunks
    (torch.bfloat16, 300, 136, 1032, 7, 0, "none"),          # general mainloop, ragged
    (torch.float32, 260, 64, 520, 9, 256, "random10"),       # fp32 matrix cores, 2 chunks
    (torch.bfloat16, 130, 128, 1280, 100, 0, "random10"),    # K > 64: the 256-thread row kernel
]
KINDS = {
    "mix": (0.5, dict()),
    "pure_reverse": (1.0, dict()),
    "every_option": (0.4, dict(tau_rows=True, partial_mass=True, labels=True, ce_weight=0.3)),
}


@pytest.mark.parametrize("kind", sorted(KINDS))
@pytest.mark.parametrize("dtype,T,d,V,K,chunk,mask", SHAPES)
def test_reverse_matches_the_oracle(kind, dtype, T, d, V, K, chunk, mask):
    r, opt = KINDS[kind]
    inp = with_duplicates(G.make_topk(T, d, V, K, dtype, tau=1.2, mask=mask, number=71, g="normal"))
    if opt:
        inp = G.add_topk_options(inp, number=71, **opt)
    say(f"reverse {kind} r={r} T={T} d={d} V={V} K={K} chunk={chunk} {dtype}")
    check(run_rev(inp, r, chunk_rows=chunk), inp, r, dtype)


def test_reverse_in_the_single_call():
    inp = with_duplicates(G.make_topk(900, 384, 1280, 16, torch.bfloat16, tau=0.9, mask="random10", number=72,
                                      g="normal"))
    inp = G.add_topk_options(inp, number=72, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.2)
    say("reverse r=0.6, every option, single call, 4 chunks")
    check(run_rev(inp, 0.6, chunk_rows=256, one_call=True), inp, 0.6, torch.bfloat16)
    # one chunk: the same bits as the forward and backward calls
    one, two = run_rev(inp, 0.6, one_call=True), run_rev(inp, 0.6)
    for k in one:
        np.testing.assert_array_equal(one[k], two[k], err_msg=k)


def test_zero_weight_gives_the_plain_bits():
    inp = G.make_topk(520, 256, 1288, 12, torch.bfloat16, tau=1.7, mask="random10", number=73, g="normal")
    say("rev_weight 0 vs plain call")
    a, b = run_rev(inp, 0.0), run_rev(inp, 0.0)
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, inp["tau"], want_z_topk=True)
    dH, dW = kd.topk_kl_backward(H, W, I, A, M, inp["tau"], lse, g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a["kl"], kl.cpu().double().numpy())
    np.testing.assert_array_equal(a["dW"], dW.cpu().double().numpy())
    np.testing.assert_array_equal(a["dW"], b["dW"])


def test_head_slice_with_reverse_and_every_option():
    inp = G.make_topk(512, 3072, 128256, 64, torch.bfloat16, tau=1.0, number=74, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.25, number=74)
    say("head slice T=512 d=3072 V=128256 K=64, reverse r=0.3 and every option")
    check(run_rev(inp, 0.3), inp, 0.3, torch.bfloat16)


def test_autograd_with_reverse():
    inp = G.make_topk(600, 256, 1288, 16, torch.bfloat16, tau=1.3, mask="random10", number=75, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, number=75)
    say("topk_kl autograd, rev_weight 0.7")
    H, W = dev(inp["H"]).requires_grad_(True), dev(inp["W"]).requires_grad_(True)
    kl = kd.topk_kl(H, W, dev(inp["I"]), dev(inp["A"]), dev(inp["mask"]), inp["tau"], chunk_rows=256,
                    tau_rows=dev(inp["tau_rows"]), rev_weight=0.7)
    (kl * dev(inp["g"])).sum().backward()
    torch.cuda.synchronize()
    kw = dict(tau_rows=inp["tau_rows"], rev_weight=0.7)
    want, _, _ = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], **kw)
    dH, dW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], **kw)
    v = inp["mask"].numpy() != 0
    assert_kl(kl.detach().cpu().double().numpy(), want, torch.bfloat16, v)
    assert_grad(H.grad.cpu().double().numpy(), dH, torch.bfloat16, "dH")
    assert_grad(W.grad.cpu().double().numpy(), dW, torch.bfloat16, "dW")
