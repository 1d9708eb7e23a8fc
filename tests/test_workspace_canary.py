"""No call writes outside its workspace: a guard pattern before and after the
caller's workspace must be untouched after every call family (the forward,
the backward over several chunks, the single call, the options, the
vocabulary shards, and the full-vocabulary calls), on the direct-load path
(bf16) and the general one (fp32)."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

FRONT, BACK, PATTERN = 4096, 65536, 0xA5


class Guarded:
    """A workspace of `nbytes` between two guard regions."""

    def __init__(self, nbytes):
        self.buf = torch.full((FRONT + nbytes + BACK,), PATTERN, dtype=torch.uint8, device="cuda")
        self.ws = self.buf[FRONT:FRONT + nbytes]
        assert self.ws.data_ptr() % 256 == 0

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.buf[:FRONT] == PATTERN).all()) and bool((self.buf[-BACK:] == PATTERN).all())


CASES = [(torch.bfloat16, 700, 384, 1280, 16), (torch.float32, 300, 136, 1032, 7)]


@pytest.mark.parametrize("dtype,T,d,V,K", CASES)
def test_topk_calls_stay_inside_their_workspace(dtype, T, d, V, K):
    inp = G.make_topk(T, d, V, K, dtype, tau=1.3, mask="random10", number=70, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.3, number=70)
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    tr, tl, y = (dev(inp[k]) for k in ("tau_rows", "teacher_lse", "labels"))
    tau = inp["tau"]
    kl, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    z = torch.empty(T, K, device="cuda")
    dH, dW = torch.empty_like(H), torch.empty(d, V, device="cuda")
    say(f"canary top-K {dtype} T={T} d={d} V={V} K={K}")
    for chunk in (0, 256):
        w = Guarded(kd.kd_topk_kl_workspace_size(T, d, V, K, dtype, chunk))
        kd.kd_topk_kl_fwd(H, W, I, A, M, tau, kl, lse, z, w.ws)
        kd.kd_topk_kl_bwd(H, W, I, A, M, tau, lse, g, dH, dW, chunk, w.ws)
        o = kd.topk_opts(tau_rows=tr, teacher_lse=tl, labels=y, ce_weight=0.3, check_indices=True)
        kd.kd_topk_kl_fwd_ex(H, W, I, A, M, tau, o, kl, lse, z, w.ws)
        kd.kd_topk_kl_bwd_ex(H, W, I, A, M, tau, o, lse, g, dH, dW, chunk, w.ws)
        assert w.intact(), f"two calls, chunk {chunk}"
        w = Guarded(kd.kd_topk_kl_fwd_bwd_workspace_size(T, d, V, K, dtype, chunk))
        kd.kd_topk_kl_fwd_bwd(H, W, I, A, M, tau, g, kl, lse, z, dH, dW, chunk, w.ws)
        kd.kd_topk_kl_fwd_bwd_ex(H, W, I, A, M, tau, o, g, kl, lse, z, dH, dW, chunk, w.ws)
        assert w.intact(), f"single call, chunk {chunk}"
    # one vocabulary shard of two
    Vs = V // 2
    Ws = W[:, Vs:].contiguous()
    w = Guarded(kd.kd_topk_kl_shard_workspace_size(T, d, V - Vs, Vs, K, dtype, 256))
    rec, trow = torch.empty(2, T, 4, device="cuda"), torch.empty(T, 2, device="cuda")
    dHs, dWs = torch.empty(T, d, device="cuda"), torch.empty(d, V - Vs, device="cuda")
    kd.kd_topk_kl_fwd_shard(H, Ws, Vs, I, A, M, tau, None, rec[1], trow, None, w.ws)
    rec[0].copy_(rec[1])
    kd.kd_topk_kl_shard_combine(rec, trow, M, kl, lse)
    kd.kd_topk_kl_bwd_shard(H, Ws, Vs, I, A, M, tau, None, lse, g, dHs, dWs, 256, w.ws)
    assert w.intact(), "shard"


@pytest.mark.parametrize("dtype,T,d,dt,V", [(torch.bfloat16, 600, 256, 384, 1288), (torch.float32, 300, 64, 96, 520)])
def test_full_vocab_calls_stay_inside_their_workspace(dtype, T, d, dt, V):
    inp = G.make_full(T, d, dt, V, dtype, mask="random10", number=71, g="normal")
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    kl, ls, lt, kr = (torch.empty(T, device="cuda") for _ in range(4))
    dH, dW = torch.empty_like(H), torch.empty(d, V, device="cuda")
    say(f"canary full {dtype} T={T} d={d} dt={dt} V={V}")
    for chunk in (0, 256):
        w = Guarded(kd.kd_full_kl_workspace_size(T, d, dt, V, dtype, chunk))
        kd.kd_full_kl_fwd(H, Ws, Ht, Wt, M, 1.0, kl, ls, lt, w.ws)
        kd.kd_full_kl_bwd(H, Ws, Ht, Wt, M, 1.0, ls, lt, g, dH, dW, chunk, w.ws)
        o = kd.full_opts(rev_weight=0.4)
        kd.kd_full_kl_fwd_ex(H, Ws, Ht, Wt, M, 1.0, o, kl, ls, lt, kr, w.ws)
        kd.kd_full_kl_bwd_ex(H, Ws, Ht, Wt, M, 1.0, o, ls, lt, kr, g, dH, dW, chunk, w.ws)
        assert w.intact(), f"two calls, chunk {chunk}"
        w = Guarded(kd.kd_full_kl_fwd_bwd_workspace_size(T, d, dt, V, dtype, chunk))
        kd.kd_full_kl_fwd_bwd(H, Ws, Ht, Wt, M, 1.0, g, kl, ls, lt, dH, dW, chunk, w.ws)
        kd.kd_full_kl_fwd_bwd_ex(H, Ws, Ht, Wt, M, 1.0, o, g, kl, ls, lt, kr, dH, dW, chunk, w.ws)
        assert w.intact(), f"single call, chunk {chunk}"
    Vs = V // 2 // 8 * 8
    Wss, Wts = Ws[:, :Vs].contiguous(), Wt[:, :Vs].contiguous()
    w = Guarded(kd.kd_full_kl_workspace_size(T, d, dt, Vs, dtype, 256))
    rec = torch.empty(1, T, 8, device="cuda")
    dHs, dWs = torch.empty(T, d, device="cuda"), torch.empty(d, Vs, device="cuda")
    kd.kd_full_kl_fwd_shard(H, Wss, Ht, Wts, M, 1.0, None, rec[0], w.ws)
    kd.kd_full_kl_shard_combine(rec, M, 0.0, kl, ls, lt, None)
    kd.kd_full_kl_bwd_shard(H, Wss, Ht, Wts, M, 1.0, None, ls, lt, None, g, dHs, dWs, 256, w.ws)
    assert w.intact(), "shard"
