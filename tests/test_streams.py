"""GPU check that every launch of a call goes to the caller's stream: the same
calls issued on a second torch stream (default priority) give the same bits
as on the default stream, for the two-call and single-call forms of both
heads.  A launch that went elsewhere would race with its neighbours."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def topk_calls(d):
    kl, lse, z = kd.topk_kl_forward(d["H"], d["W"], d["I"], d["A"], d["mask"], d["tau"], want_z_topk=True)
    dH, dW = kd.topk_kl_backward(d["H"], d["W"], d["I"], d["A"], d["mask"], d["tau"], lse, d["g"], 256)
    one = kd.topk_kl_forward_backward(d["H"], d["W"], d["I"], d["A"], d["mask"], d["tau"], d["g"], 256,
                                      want_z_topk=True)
    return [kl, lse, z, dH, dW, *one]


def full_calls(d):
    kl, ls, lt = kd.full_kl_forward(d["H"], d["Ws"], d["Ht"], d["Wt"], d["mask"], d["tau"])
    dH, dW = kd.full_kl_backward(d["H"], d["Ws"], d["Ht"], d["Wt"], d["mask"], d["tau"], ls, lt, d["g"], 256)
    one = kd.full_kl_forward_backward(d["H"], d["Ws"], d["Ht"], d["Wt"], d["mask"], d["tau"], d["g"], 256)
    return [kl, ls, lt, dH, dW, *one]


@pytest.mark.parametrize("head", ["topk", "full"])
def test_side_stream_gives_the_same_bits(head):
    if head == "topk":
        inp = G.make_topk(700, 384, 2568, 16, torch.bfloat16, tau=1.1, mask="random10", number=71, g="normal")
        calls = topk_calls
    else:
        inp = G.make_full(700, 384, 256, 2568, torch.bfloat16, tau=1.1, mask="random10", number=72, g="normal")
        calls = full_calls
    d = {k: (dev(v) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say(f"{head}: default stream vs a second stream")
    ref = [x.cpu() for x in calls(d)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = calls(d)
    s.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        np.testing.assert_array_equal(a.cpu().float().numpy(), b.float().numpy(), err_msg=f"output {i}")
