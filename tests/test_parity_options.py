"""GPU parity of the optional parts of the top-K loss (kd_topk_opts: per-token
temperature, partial-mass teacher, LM cross-entropy mix) against the fp64
oracle's topk_loss_*, through the _ex calls of the C-ABI.

Options only change the prep kernel's per-row constants and the weights of
the support entries; so an option that changes nothing (per-row temperatures
all equal to tau, labels with weight 0) must give the plain call's bits.
"""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, run_topk, say

pytestmark = pytest.mark.gpu

OPTS = ("tau_rows", "teacher_lse", "labels")


def options(inp):
    o = {k: dev(inp[k]) for k in OPTS if k in inp}
    if "labels" in inp:
        o["ce_weight"] = inp["ce_weight"]
    return o


def run_opts(inp, chunk_rows=0, one_call=False):
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    tau, o = inp["tau"], options(inp)
    if one_call:
        kl, lse, z, dH, dW = kd.topk_kl_forward_backward(H, W, I, A, M, tau, g, chunk_rows, want_z_topk=True, **o)
    else:
        kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, want_z_topk=True, **o)
        dH, dW = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, chunk_rows, **o)
    torch.cuda.synchronize()
    return {k: v.cpu().double().numpy() for k, v in dict(kl=kl, lse=lse, z=z, dH=dH, dW=dW).items()}


def oracle_kw(inp):
    kw = {k: inp[k] for k in OPTS if k in inp}
    if "labels" in inp:
        kw["ce_weight"] = inp["ce_weight"]
    return kw


def check(got, inp, dtype):
    kw = oracle_kw(inp)
    kl, lse, z = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], **kw)
    dH, dW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], **kw)
    T = kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, dtype, v)
    assert_lse(got["lse"], lse, dtype, v)
    np.testing.assert_allclose(got["z"][v], z[v], rtol=1e-4 if dtype == torch.bfloat16 else 1e-5, atol=1e-5)
    for k in ("kl", "lse", "z", "dH"):
        assert np.all(got[k][~v] == 0), k
    assert_grad(got["dH"], dH, dtype, "dH")
    assert_grad(got["dW"], dW, dtype, "dW")


SHAPES = [
    (torch.bfloat16, 700, 384, 2568, 24, 256, "random10"),   # direct-load, shifted last tile, 3 chunks
    (torch.bfloat16, 300, 136, 1032, 7, 0, "none"),          # general mainloop, ragged
    (torch.float32, 260, 64, 520, 9, 256, "random10"),       # fp32 matrix cores, 2 chunks
]
KINDS = {
    "tau_rows": dict(tau_rows=True),
    "partial_mass": dict(partial_mass=True),
    "ce_mix": dict(labels=True, ce_weight=0.3),
    "pure_ce": dict(labels=True, ce_weight=1.0),
    "all": dict(tau_rows=True, partial_mass=True, labels=True, ce_weight=0.45),
}


@pytest.mark.parametrize("kind", sorted(KINDS))
@pytest.mark.parametrize("dtype,T,d,V,K,chunk,mask", SHAPES)
def test_options_match_the_oracle(kind, dtype, T, d, V, K, chunk, mask):
    inp = G.make_topk(T, d, V, K, dtype, tau=1.2, mask=mask, number=31, g="normal")
    inp = G.add_topk_options(inp, number=31, **KINDS[kind])
    say(f"options {kind} T={T} d={d} V={V} K={K} chunk={chunk} {dtype}")
    check(run_opts(inp, chunk_rows=chunk), inp, dtype)


@pytest.mark.parametrize("kind", ["partial_mass", "all"])
def test_options_in_the_single_call(kind):
    inp = G.make_topk(900, 384, 1280, 16, torch.bfloat16, tau=0.9, mask="random10", number=32, g="normal")
    inp = G.add_topk_options(inp, number=32, **KINDS[kind])
    say(f"options {kind}, single call, 4 chunks")
    got = run_opts(inp, chunk_rows=256, one_call=True)
    check(got, inp, torch.bfloat16)
    # one chunk: the same bits as the forward and backward calls
    one, two = run_opts(inp, one_call=True), run_opts(inp)
    for k in one:
        np.testing.assert_array_equal(one[k], two[k], err_msg=k)


def test_neutral_options_give_the_plain_bits():
    inp = G.make_topk(520, 256, 1288, 12, torch.bfloat16, tau=1.7, mask="random10", number=33, g="normal")
    say("neutral options vs plain call")
    plain = run_topk(inp, chunk_rows=256)
    same = dict(inp)
    same["tau_rows"] = torch.full((520,), 1.7, dtype=torch.float32)
    same["labels"] = torch.zeros(520, dtype=torch.int32)
    same["ce_weight"] = 0.0
    got = run_opts(same, chunk_rows=256)
    for k in plain:
        np.testing.assert_array_equal(got[k], plain[k], err_msg=k)


def test_label_entry_leaves_z_topk_alone():
    # the label is an extra support entry; z_topk still holds the K cached ones
    inp = G.make_topk(400, 128, 1024, 8, torch.bfloat16, tau=1.0, number=34, g="normal")
    inp = G.add_topk_options(inp, labels=True, ce_weight=0.6, number=34)
    say("z_topk with a CE label")
    got, plain = run_opts(inp), run_topk(inp)
    np.testing.assert_array_equal(got["z"], plain["z"])
    np.testing.assert_array_equal(got["lse"], plain["lse"])


def test_head_slice_with_every_option():
    inp = G.make_topk(512, 3072, 128256, 64, torch.bfloat16, tau=1.0, number=35, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.25, number=35)
    say("head slice T=512 d=3072 V=128256 K=64, every option")
    check(run_opts(inp), inp, torch.bfloat16)


def test_head_t4096_every_option_sampled_rows():
    p = G.PRESETS["head_topk_t4096"]
    inp = G.add_topk_options(G.make_preset(p, g="normal"), tau_rows=True, partial_mass=True, labels=True,
                             ce_weight=0.25, number=p.number)
    say("head T=4096, every option, sampled rows")
    got = run_opts(inp)
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set(rng.choice(4096, 40, replace=False).tolist()) | {0, 255, 256, 4095}))
    kl, lse, z, dH = O.topk_loss_rows(inp["H"], inp["W"], inp["I"], inp["A"], None, p.tau, inp["g"], rows,
                                      **oracle_kw(inp))
    assert_kl(got["kl"][rows], kl, torch.bfloat16)
    assert_lse(got["lse"][rows], lse, torch.bfloat16)
    np.testing.assert_allclose(got["z"][rows], z, rtol=1e-4, atol=1e-5)
    assert_grad(got["dH"][rows], dH, torch.bfloat16, "dH rows")
    assert np.all(np.isfinite(got["dW"]))
