"""GPU parity when most rows are masked: the forward runs in chunks of the
default chunk size and the backward in chunks of chunk_rows, over compacted
rows, so chunks that lie wholly past the valid rows launch with nothing to do
and a last partial chunk gets a launch shape sized to its own rows.  Every
output is checked against the fp64 oracle, for both heads and both call
forms (forward then backward, and the single call).
"""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, run_full, run_topk, say

pytestmark = pytest.mark.gpu

T, N_MASKED = 9000, 5400  # 3600 valid rows: forward chunks 2 and 3 of 4096 rows are empty


def valid(inp):
    return inp["mask"].numpy() != 0


def topk_inputs():
    return G.make_topk(T, 256, 1288, 12, torch.bfloat16, tau=1.1, mask="random10", n_masked=N_MASKED, number=41,
                       g="normal")


def check_topk(got, inp, want):
    v = valid(inp)
    assert_kl(got["kl"], want["kl"], torch.bfloat16, v)
    assert_lse(got["lse"], want["lse"], torch.bfloat16, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["lse"][~v] == 0) and np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], want["dH"], torch.bfloat16, "dH")
    assert_grad(got["dW"], want["dW"], torch.bfloat16, "dW")


@pytest.fixture(scope="module")
def topk_case():
    inp = topk_inputs()
    kl, lse, z = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"])
    dH, dW = O.topk_kl_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"])
    return inp, dict(kl=kl, lse=lse, z=z, dH=dH, dW=dW)


@pytest.mark.parametrize("chunk", [1024, 3840])
def test_topk_two_calls_with_empty_chunks(topk_case, chunk):
    inp, want = topk_case
    say(f"top-K T={T} with {N_MASKED} masked rows, chunk_rows={chunk}")
    check_topk(run_topk(inp, want_z=False, chunk_rows=chunk), inp, want)


def test_topk_single_call_with_empty_chunks(topk_case):
    inp, want = topk_case
    say(f"top-K single call T={T} with {N_MASKED} masked rows, chunk_rows=1024")
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    kl, lse, z, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, M, inp["tau"], g, 1024, want_z_topk=True)
    torch.cuda.synchronize()
    got = {k: x.cpu().double().numpy() for k, x in dict(kl=kl, lse=lse, z=z, dH=dH, dW=dW).items()}
    check_topk(got, inp, want)
    v = valid(inp)
    np.testing.assert_allclose(got["z"][v], want["z"][v], rtol=1e-4, atol=1e-5)


@pytest.fixture(scope="module")
def full_case():
    inp = G.make_full(T, 256, 128, 1288, torch.bfloat16, tau=0.9, mask="random10", number=42, g="normal",
                      n_masked=N_MASKED)
    kl, ls, lt = O.full_kl_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"])
    dH, dW = O.full_kl_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], inp["g"])
    return inp, dict(kl=kl, lse_s=ls, lse_t=lt, dH=dH, dW=dW)


def check_full(got, inp, want):
    v = valid(inp)
    assert_kl(got["kl"], want["kl"], torch.bfloat16, v)
    assert_lse(got["lse_s"], want["lse_s"], torch.bfloat16, v)
    assert_lse(got["lse_t"], want["lse_t"], torch.bfloat16, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], want["dH"], torch.bfloat16, "dH")
    assert_grad(got["dW"], want["dW"], torch.bfloat16, "dWs")


def test_full_two_calls_with_empty_chunks(full_case):
    inp, want = full_case
    say(f"full T={T} with {N_MASKED} masked rows, chunk_rows=1024")
    check_full(run_full(inp, chunk_rows=1024), inp, want)


def test_full_single_call_with_empty_chunks(full_case):
    inp, want = full_case
    say(f"full single call T={T} with {N_MASKED} masked rows, chunk_rows=1024")
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    kl, ls, lt, dH, dW = kd.full_kl_forward_backward(H, Ws, Ht, Wt, M, inp["tau"], g, 1024)
    torch.cuda.synchronize()
    got = {k: x.cpu().double().numpy() for k, x in dict(kl=kl, lse_s=ls, lse_t=lt, dH=dH, dW=dW).items()}
    check_full(got, inp, want)
