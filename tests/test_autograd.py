"""GPU check of the autograd wrappers (topk_kl, full_kl): the loss sum(g * kl)
back-propagated through torch gives the fp64 oracle's dH and dW for that
per-token weight g, with W's gradient in W's dtype, and no gradient for the
teacher's tensors."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, dev, say

pytestmark = pytest.mark.gpu


def leaf(x):
    return dev(x).requires_grad_(True)


@pytest.mark.parametrize("options", [False, True])
def test_topk_kl_autograd(options):
    inp = G.make_topk(600, 256, 1288, 16, torch.bfloat16, tau=1.3, mask="random10", number=61, g="normal")
    kw = {}
    if options:
        inp = G.add_topk_options(inp, tau_rows=True, labels=True, ce_weight=0.25, number=61)
        kw = dict(tau_rows=dev(inp["tau_rows"]), labels=dev(inp["labels"]), ce_weight=inp["ce_weight"])
    say(f"topk_kl autograd options={options}")
    H, W = leaf(inp["H"]), leaf(inp["W"])
    kl = kd.topk_kl(H, W, dev(inp["I"]), dev(inp["A"]), dev(inp["mask"]), inp["tau"], chunk_rows=256, **kw)
    (kl * dev(inp["g"])).sum().backward()
    torch.cuda.synchronize()
    okw = {k: inp[k] for k in ("tau_rows", "labels", "ce_weight") if k in inp}
    want_kl, _, _ = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], **okw)
    dH, dW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], **okw)
    v = inp["mask"].numpy() != 0
    assert_kl(kl.detach().cpu().double().numpy(), want_kl, torch.bfloat16, v)
    assert H.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    assert_grad(H.grad.cpu().double().numpy(), dH, torch.bfloat16, "dH")
    assert_grad(W.grad.cpu().double().numpy(), dW, torch.bfloat16, "dW")


def test_full_kl_autograd():
    inp = G.make_full(600, 256, 384, 1288, torch.bfloat16, tau=0.8, mask="random10", number=62, g="normal")
    say("full_kl autograd")
    H, Ws = leaf(inp["H"]), leaf(inp["Ws"])
    Ht, Wt = leaf(inp["Ht"]), leaf(inp["Wt"])
    kl = kd.full_kl(H, Ws, Ht, Wt, dev(inp["mask"]), inp["tau"], chunk_rows=256)
    (kl * dev(inp["g"])).sum().backward()
    torch.cuda.synchronize()
    want_kl, _, _ = O.full_kl_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"])
    dH, dW = O.full_kl_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], inp["g"])
    v = inp["mask"].numpy() != 0
    assert_kl(kl.detach().cpu().double().numpy(), want_kl, torch.bfloat16, v)
    assert_grad(H.grad.cpu().double().numpy(), dH, torch.bfloat16, "dH")
    assert_grad(Ws.grad.cpu().double().numpy(), dW, torch.bfloat16, "dWs")
    assert Ht.grad is None and Wt.grad is None
    assert np.all(np.isfinite(H.grad.cpu().float().numpy()))
