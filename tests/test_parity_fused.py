"""GPU parity of the single-call forward + backward (kd_topk_kl_fwd_bwd,
kd_full_kl_fwd_bwd).

Each computes what its forward call followed by its backward call computes,
from the chunk's kept fp32 logits instead of a second projection.  Top-K:
when one chunk holds every row, the vocabulary splits and every formula are
the same as in the two-call path, so the outputs must be bit-identical to it;
with several chunks the split count per chunk differs and the outputs are
checked against the fp64 oracle instead.  Full vocabulary: the single call
takes each head through its own 256-column tiles, so it is checked against
the oracle (and the two-call path) within the tolerances.
"""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, run_full, run_topk, say

pytestmark = pytest.mark.gpu


def run_fused(inp, chunk_rows=0, want_z=True):
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    kl, lse, z, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, M, inp["tau"], g, chunk_rows, want_z_topk=want_z)
    torch.cuda.synchronize()
    return dict(kl=kl.cpu().double().numpy(), lse=lse.cpu().double().numpy(),
                z=None if z is None else z.cpu().double().numpy(),
                dH=dH.cpu().double().numpy(), dW=dW.cpu().double().numpy())


@pytest.mark.parametrize("dtype,T,d,V,K,tau,mask", [
    (torch.bfloat16, 512, 3072, 128256, 64, 1.0, "none"),     # the output head, direct-load kernels
    (torch.bfloat16, 700, 384, 2568, 16, 1.3, "random10"),    # direct-load, last vocab tile shifted, masked
    (torch.bfloat16, 300, 136, 1032, 7, 1.0, "none"),         # general mainloop, ragged everything
    (torch.float32, 513, 64, 520, 33, 0.7, "random10"),       # fp32 matrix cores
])
def test_single_chunk_matches_two_calls_bitwise(dtype, T, d, V, K, tau, mask):
    inp = G.make_topk(T, d, V, K, dtype, tau=tau, mask=mask, number=21, g="normal")
    say(f"fused vs two calls T={T} d={d} V={V} K={K} {dtype}")
    two = run_topk(inp)
    one = run_fused(inp)
    for k in ("kl", "lse", "z", "dH", "dW"):
        np.testing.assert_array_equal(one[k], two[k], err_msg=k)


@pytest.mark.parametrize("dtype,T,d,V,K,chunk,mask", [
    (torch.bfloat16, 900, 384, 1280, 24, 256, "random10"),    # 4 chunks (last ragged), direct-load
    (torch.bfloat16, 600, 200, 2056, 5, 256, "none"),         # general mainloop, 3 chunks
    (torch.float32, 520, 64, 1032, 9, 256, "random10"),       # fp32, 3 chunks
])
def test_several_chunks_match_the_oracle(dtype, T, d, V, K, chunk, mask):
    inp = G.make_topk(T, d, V, K, dtype, tau=1.2, mask=mask, number=22, g="normal")
    say(f"fused chunks={chunk} T={T} d={d} V={V} K={K} {dtype}")
    got = run_fused(inp, chunk_rows=chunk)
    kl, lse, z = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"])
    dH, dW = O.topk_kl_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"])
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse"], lse, dtype, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["lse"][~v] == 0) and np.all(got["dH"][~v] == 0)
    np.testing.assert_allclose(got["z"][v], z[v], rtol=1e-4, atol=1e-5)
    assert np.all(got["z"][~v] == 0)
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dW")


def test_all_rows_masked_and_empty_batch():
    inp = G.make_topk(300, 64, 520, 4, torch.bfloat16, number=23, g="normal")
    inp["mask"] = torch.zeros(300, dtype=torch.uint8)
    say("fused, every row masked")
    got = run_fused(inp, chunk_rows=256)
    for k in ("kl", "lse", "z", "dH", "dW"):
        assert np.all(got[k] == 0), k
    say("fused, T = 0")
    H = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.randn(64, 520, device="cuda").to(torch.bfloat16)
    I = torch.empty(0, 4, dtype=torch.int32, device="cuda")
    A = torch.empty(0, 4, device="cuda")
    g = torch.empty(0, device="cuda")
    kl, lse, z, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, None, 1.0, g)
    torch.cuda.synchronize()
    assert kl.numel() == 0 and dH.numel() == 0 and torch.all(dW == 0)


# ---------------------------------------------------------------- full vocabulary
def run_full_fused(inp, chunk_rows=0):
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    kl, ls, lt, dH, dW = kd.full_kl_forward_backward(H, Ws, Ht, Wt, M, inp["tau"], g, chunk_rows)
    torch.cuda.synchronize()
    return dict(kl=kl.cpu().double().numpy(), lse_s=ls.cpu().double().numpy(), lse_t=lt.cpu().double().numpy(),
                dH=dH.cpu().double().numpy(), dW=dW.cpu().double().numpy())


def check_full(got, inp, dtype):
    kl, lse_s, lse_t = O.full_kl_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"])
    dH, dW = O.full_kl_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], inp["g"])
    T = kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse_s"], lse_s, dtype, v)
    assert_lse(got["lse_t"], lse_t, dtype, v)
    for k in ("kl", "lse_s", "lse_t", "dH"):
        assert np.all(got[k][~v] == 0), k
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dWs")


# The single call takes each head through the 256-column top-K tiles and the
# KL terms from the exact normalisers, so it matches the two-call path (and
# the oracle) within rounding, not bit for bit.
@pytest.mark.parametrize("dtype,T,d,dt,V,tau,mask", [
    (torch.bfloat16, 512, 3072, 4096, 128256, 1.0, "none"),   # the heads of the full-vocabulary workload
    (torch.bfloat16, 700, 384, 256, 1288, 1.3, "random10"),   # direct-load, ragged last vocabulary tile, masked
    (torch.bfloat16, 300, 136, 72, 1032, 1.0, "none"),        # general mainloop, ragged everything
    (torch.float32, 513, 64, 128, 520, 0.8, "random10"),      # fp32 matrix cores
])
def test_full_single_chunk_matches_the_oracle_and_two_calls(dtype, T, d, dt, V, tau, mask):
    inp = G.make_full(T, d, dt, V, dtype, tau=tau, mask=mask, number=26, g="normal")
    say(f"full fused vs oracle and two calls T={T} d={d} dt={dt} V={V} {dtype}")
    one = run_full_fused(inp)
    check_full(one, inp, dtype)
    two = run_full(inp)
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(one["kl"], two["kl"], dtype, v)
    assert_grad(one["dW"], two["dW"], dtype, "dWs vs two calls")


def test_full_single_call_is_deterministic():
    inp = G.make_full(600, 256, 384, 2056, torch.bfloat16, mask="random10", number=29, g="normal")
    say("full fused determinism")
    a, b = run_full_fused(inp, chunk_rows=256), run_full_fused(inp, chunk_rows=256)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("dtype,T,d,dt,V,chunk,mask", [
    (torch.bfloat16, 900, 256, 384, 1288, 256, "random10"),   # 4 chunks (last ragged), direct-load
    (torch.bfloat16, 600, 200, 136, 2056, 256, "none"),       # general mainloop, 3 chunks
    (torch.float32, 520, 64, 40, 1032, 256, "random10"),      # fp32, 3 chunks
])
def test_full_several_chunks_match_the_oracle(dtype, T, d, dt, V, chunk, mask):
    inp = G.make_full(T, d, dt, V, dtype, tau=1.4, mask=mask, number=27, g="normal")
    say(f"full fused chunks={chunk} T={T} d={d} dt={dt} V={V} {dtype}")
    check_full(run_full_fused(inp, chunk_rows=chunk), inp, dtype)


def test_full_all_rows_masked_and_empty_batch():
    inp = G.make_full(300, 64, 40, 520, torch.bfloat16, number=28, g="normal")
    inp["mask"] = torch.zeros(300, dtype=torch.uint8)
    say("full fused, every row masked")
    got = run_full_fused(inp, chunk_rows=256)
    for k in ("kl", "lse_s", "lse_t", "dH", "dW"):
        assert np.all(got[k] == 0), k
    say("full fused, T = 0")
    H = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    Ht = torch.empty(0, 40, dtype=torch.bfloat16, device="cuda")
    Ws = torch.randn(64, 520, device="cuda").to(torch.bfloat16)
    Wt = torch.randn(40, 520, device="cuda").to(torch.bfloat16)
    g = torch.empty(0, device="cuda")
    kl, ls, lt, dH, dW = kd.full_kl_forward_backward(H, Ws, Ht, Wt, None, 1.0, g)
    torch.cuda.synchronize()
    assert kl.numel() == 0 and dH.numel() == 0 and torch.all(dW == 0)
