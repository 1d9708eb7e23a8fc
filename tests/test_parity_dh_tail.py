"""GPU parity of dH when the vocabulary is a multiple of 32 but not of 128
(V = 16032, a head of 128256 columns split 8 ways, is one).  dH's direct-load
ring then contracts V rounded up to 128 over the dZ chunk's zeroed tail, with
W's stages past V clamped to its last one.  Both heads, both call forms,
several backward chunks (the tail must stay zero from chunk to chunk), and
vocabularies under one 256-column tile.
"""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import dev, run_full, run_topk, say
from tests.test_parity_full import check_all, oracle_all
from tests.test_parity_options import check, run_opts

pytestmark = pytest.mark.gpu

SHAPES = [
    # T, d, V, chunk_rows
    (700, 384, 1312, 256),  # V % 128 = 32: three chunks, direct-load forward tiles
    (600, 256, 2400, 256),  # V % 128 = 96
    (300, 256, 160, 256),   # under one tile: V % 128 = 32, rounded up to 256 = the chunk's width
]


@pytest.mark.parametrize("T,d,V,chunk", SHAPES)
@pytest.mark.parametrize("one_call", [False, True])
def test_topk(T, d, V, chunk, one_call):
    inp = G.make_topk(T, d, V, 12, torch.bfloat16, tau=1.1, mask="random10", number=91, g="normal")
    say(f"top-K dH tail T={T} d={d} V={V} chunk={chunk} one_call={one_call}")
    check(run_opts(inp, chunk_rows=chunk, one_call=one_call), inp, torch.bfloat16)


@pytest.mark.parametrize("T,d,V,chunk", SHAPES)
def test_full_two_calls(T, d, V, chunk):
    inp = G.make_full(T, d, 128, V, torch.bfloat16, tau=0.9, mask="random10", number=92, g="normal")
    say(f"full dH tail T={T} d={d} V={V} chunk={chunk}")
    check_all(run_full(inp, chunk_rows=chunk), oracle_all(inp), inp, torch.bfloat16)


@pytest.mark.parametrize("T,d,V,chunk", SHAPES)
def test_full_single_call(T, d, V, chunk):
    inp = G.make_full(T, d, 128, V, torch.bfloat16, tau=0.9, mask="random10", number=93, g="normal")
    say(f"full single call dH tail T={T} d={d} V={V} chunk={chunk}")
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    kl, ls, lt, dH, dW = kd.full_kl_forward_backward(H, Ws, Ht, Wt, M, inp["tau"], g, chunk)
    torch.cuda.synchronize()
    got = {k: x.cpu().double().numpy() for k, x in dict(kl=kl, lse_s=ls, lse_t=lt, dH=dH, dW=dW).items()}
    check_all(got, oracle_all(inp), inp, torch.bfloat16)


def test_stale_workspace_does_not_leak_into_dh():
    # a forward call leaves its partials where the backward's chunk buffers
    # lie; the backward must clear the dZ tail itself
    inp = G.make_topk(700, 384, 1312, 12, torch.bfloat16, tau=1.0, number=94, g="normal")
    H, W, I, A, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "g"))
    say("top-K dH tail after a workspace filled with NaN")
    ws = torch.full((kd.kd_topk_kl_workspace_size(700, 384, 1312, 12, torch.bfloat16, 256),), 0xFF,
                    dtype=torch.uint8, device="cuda")  # bytes 0xFF: NaN in bf16 and fp32
    kl, lse, _ = kd.topk_kl_forward(H, W, I, A, None, 1.0, workspace=ws)
    dH, dW = kd.topk_kl_backward(H, W, I, A, None, 1.0, lse, g, 256, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dH).all()) and bool(torch.isfinite(dW).all())
    ref = run_topk(inp, want_z=False, chunk_rows=256)
    np.testing.assert_array_equal(dH.cpu().double().numpy(), ref["dH"])
