"""GPU parity of the full-vocabulary options (kd_full_opts: KL mixing with
the reverse KL, per-token temperature) against the fp64 oracle's
full_loss_*, through the _ex calls of the C-ABI, on both mainloops, fp32,
the chunked backward and the single call.  Options that change nothing must
give the plain call's bits."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, run_full, say

pytestmark = pytest.mark.gpu


def run_opts(inp, chunk_rows=0, one_call=False):
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    o = dict(tau_rows=dev(inp.get("tau_rows")), rev_weight=inp.get("rev_weight", 0.0))
    if one_call:
        kl, ls, lt, kr, dH, dW = kd.full_kl_forward_backward(H, Ws, Ht, Wt, M, inp["tau"], g, chunk_rows,
                                                             want_kl_rev=True, **o)
    else:
        kl, ls, lt, kr = kd.full_kl_forward(H, Ws, Ht, Wt, M, inp["tau"], want_kl_rev=True, **o)
        dH, dW = kd.full_kl_backward(H, Ws, Ht, Wt, M, inp["tau"], ls, lt, g, chunk_rows, kl_rev=kr, **o)
    torch.cuda.synchronize()
    out = dict(kl=kl, lse_s=ls, lse_t=lt, kl_rev=kr, dH=dH, dW=dW)
    return {k: v.cpu().double().numpy() for k, v in out.items()}


def check(got, inp, dtype):
    kw = dict(tau_rows=inp.get("tau_rows"), rev_weight=inp.get("rev_weight", 0.0))
    a = (inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"])
    kl, ls, lt, kr = O.full_loss_forward(*a, **kw)
    dH, dW = O.full_loss_backward(*a, inp["g"], **kw)
    T = kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, dtype, v)
    assert_kl(got["kl_rev"], kr, dtype, v)
    assert_lse(got["lse_s"], ls, dtype, v)
    assert_lse(got["lse_t"], lt, dtype, v)
    for k in ("kl", "lse_s", "lse_t", "kl_rev", "dH"):
        assert np.all(got[k][~v] == 0), k
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dWs")


SHAPES = [
    (torch.bfloat16, 700, 384, 256, 1288, 256, "random10"),   # direct-load, ragged last tile, 3 chunks
    (torch.bfloat16, 300, 136, 72, 1032, 0, "none"),          # general mainloop
    (torch.float32, 260, 64, 40, 520, 256, "random10"),       # fp32 matrix cores, 2 chunks
]
KINDS = {
    "mix": dict(rev_weight=0.35),
    "reverse": dict(rev_weight=1.0),
    "tau_rows": dict(tau_rows=True),
    "both": dict(tau_rows=True, rev_weight=0.6),
}


@pytest.mark.parametrize("kind", sorted(KINDS))
@pytest.mark.parametrize("dtype,T,d,dt,V,chunk,mask", SHAPES)
def test_full_options_match_the_oracle(kind, dtype, T, d, dt, V, chunk, mask):
    inp = G.make_full(T, d, dt, V, dtype, tau=1.1, mask=mask, number=41, g="normal")
    inp = G.add_full_options(inp, number=41, **KINDS[kind])
    say(f"full options {kind} T={T} d={d} dt={dt} V={V} chunk={chunk} {dtype}")
    check(run_opts(inp, chunk_rows=chunk), inp, dtype)


def test_full_options_in_the_single_call():
    inp = G.make_full(900, 256, 384, 1288, torch.bfloat16, tau=0.8, mask="random10", number=42, g="normal")
    inp = G.add_full_options(inp, tau_rows=True, rev_weight=0.5, number=42)
    say("full options, single call, 4 chunks")
    check(run_opts(inp, chunk_rows=256, one_call=True), inp, torch.bfloat16)
    check(run_opts(inp, one_call=True), inp, torch.bfloat16)


def test_full_neutral_options_give_the_plain_bits():
    inp = G.make_full(520, 256, 128, 1288, torch.bfloat16, tau=1.7, mask="random10", number=43, g="normal")
    say("full neutral options vs plain call")
    plain = run_full(inp, chunk_rows=256)
    same = dict(inp, tau_rows=torch.full((520,), 1.7, dtype=torch.float32), rev_weight=0.0)
    got = run_opts(same, chunk_rows=256)
    for k in plain:
        np.testing.assert_array_equal(got[k], plain[k], err_msg=k)


def test_full_head_slice_with_every_option():
    inp = G.make_full(256, 3072, 4096, 128256, torch.bfloat16, number=44, g="normal")
    inp = G.add_full_options(inp, tau_rows=True, rev_weight=0.4, number=44)
    say("full head slice T=256 d=3072 dt=4096 V=128256, every option")
    check(run_opts(inp), inp, torch.bfloat16)
