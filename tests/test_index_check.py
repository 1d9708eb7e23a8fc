"""The index range check on request (kd_topk_opts.check_indices): a cached
index or a label of a valid row outside [0, V) makes the call return
KD_ERR_INDEX_OUT_OF_RANGE after the teacher preparation, with nothing more
enqueued; masked rows are not checked; with every index in range the call
gives the bits of the unchecked call.  "Efficient Knowledge Distillation for
LLMs: Offline Top-K Logits and a Fused Chunked KL Loss", §3 "Offline
distillation": the cache holds K vocabulary indices per position."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

KD_ERR_INDEX_OUT_OF_RANGE = 5


def inputs():
    inp = G.make_topk(300, 128, 1280, 16, torch.bfloat16, tau=1.2, mask="random10", number=60, g="normal")
    return {k: (dev(v) if torch.is_tensor(v) else v) for k, v in inp.items()}


def calls(inp, I, **opt):
    """The three top-K call families on the same inputs; outputs pre-filled with a sentinel."""
    H, W, A, M, g, tau = inp["H"], inp["W"], inp["A"], inp["mask"], inp["g"], inp["tau"]
    T, K = I.shape
    out = {}
    kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, want_z_topk=True, **opt)
    out["fwd"] = (kl, lse, z)
    out["bwd"] = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, **opt)
    out["one"] = kd.topk_kl_forward_backward(H, W, I, A, M, tau, g, want_z_topk=True, **opt)
    torch.cuda.synchronize()
    return {k: [x.float().cpu().numpy() for x in v if x is not None] for k, v in out.items()}


def test_in_range_indices_give_the_unchecked_bits():
    inp = inputs()
    say("index check: all indices in range")
    a = calls(inp, inp["I"])
    b = calls(inp, inp["I"], check_indices=True)
    for k in a:
        for x, y in zip(a[k], b[k]):
            np.testing.assert_array_equal(x, y, err_msg=k)


def test_bad_indices_in_masked_rows_are_not_checked():
    inp = inputs()
    I = inp["I"].clone()
    m = inp["mask"] == 0
    I[m, 0] = 1280 + 7
    I[m, 1] = -2
    say("index check: out-of-range indices only in masked rows")
    calls(inp, I, check_indices=True)


@pytest.mark.parametrize("bad", [1280, 1280 + 999, -1, -(1 << 30)])
def test_out_of_range_index_in_a_valid_row_is_reported(bad):
    inp = inputs()
    I = inp["I"].clone()
    row = int(torch.nonzero(inp["mask"])[5])
    I[row, 3] = bad
    H, W, A, M, g, tau = inp["H"], inp["W"], inp["A"], inp["mask"], inp["g"], inp["tau"]
    T, K = I.shape
    ws = torch.empty(kd.kd_topk_kl_fwd_bwd_workspace_size(T, 128, 1280, K, H.dtype), dtype=torch.uint8, device="cuda")
    o = kd.topk_opts(check_indices=True)
    kl = torch.full((T,), 7.0, device="cuda")
    lse = torch.full((T,), 7.0, device="cuda")
    dH = torch.full_like(H, 7.0)
    dW = torch.full((128, 1280), 7.0, device="cuda")
    say(f"index check: index {bad} in valid row {row}")
    for name, call in (
            ("fwd", lambda: kd.kd_topk_kl_fwd_ex(H, W, I, A, M, tau, o, kl, lse, None, ws)),
            ("bwd", lambda: kd.kd_topk_kl_bwd_ex(H, W, I, A, M, tau, o, lse, g, dH, dW, 0, ws)),
            ("one", lambda: kd.kd_topk_kl_fwd_bwd_ex(H, W, I, A, M, tau, o, g, kl, lse, None, dH, dW, 0, ws))):
        with pytest.raises(kd.KDError) as e:
            call()
        assert e.value.status == KD_ERR_INDEX_OUT_OF_RANGE, name
        assert "outside [0, V)" in str(e.value)
        torch.cuda.synchronize()
        # nothing past the check was enqueued: the outputs keep their sentinel
        assert bool((kl == 7.0).all()) and bool((lse == 7.0).all()), name
        assert bool((dH == 7.0).all()) and bool((dW == 7.0).all()), name


def test_out_of_range_label_is_reported():
    inp = inputs()
    T = inp["I"].shape[0]
    labels = inp["I"][:, 0].clone()
    row = int(torch.nonzero(inp["mask"])[0])
    labels[row] = 1280
    say("index check: a label out of range")
    with pytest.raises(kd.KDError) as e:
        kd.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], labels=labels,
                           ce_weight=0.5, check_indices=True)
    assert e.value.status == KD_ERR_INDEX_OUT_OF_RANGE
    torch.cuda.synchronize()


@pytest.mark.parametrize("fill", [0xFF, 0x01])
def test_the_check_does_not_depend_on_the_workspace_contents(fill):
    # the counter lives in the workspace and is cleared by each call: left-over
    # bytes must neither hide a bad index (0xFF: -1 + 1 = 0) nor invent one
    # (0x01: a positive count with every index in range)
    inp = inputs()
    H, W, I, A, M, tau = inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"]
    T, K = I.shape
    ws = torch.full((kd.kd_topk_kl_workspace_size(T, 128, 1280, K, H.dtype),), fill, dtype=torch.uint8, device="cuda")
    kl, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    o = kd.topk_opts(check_indices=True)
    say(f"index check with a workspace filled with {fill:#x}")
    kd.kd_topk_kl_fwd_ex(H, W, I, A, M, tau, o, kl, lse, None, ws)  # every index in range
    torch.cuda.synchronize()
    ws.fill_(fill)
    bad = I.clone()
    bad[int(torch.nonzero(M)[0]), 0] = 1280
    with pytest.raises(kd.KDError) as e:
        kd.kd_topk_kl_fwd_ex(H, W, bad, A, M, tau, o, kl, lse, None, ws)
    assert e.value.status == KD_ERR_INDEX_OUT_OF_RANGE
    torch.cuda.synchronize()
