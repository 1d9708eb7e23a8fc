"""kd_topk_kl_fwd_noalloc, the top-K forward for callers that cannot allocate,
against kd_topk_kl_fwd with a workspace on the same inputs: the two run the
same kernels in the same order, so every output must match bit for bit.  The
calls come in a row on one GPU, each smaller than the one before, so the
fixed scratch array still holds the previous call's data when the next one
starts; stale contents must not show.  Outputs are filled with NaN first, so
anything a call fails to write shows too."""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


def outputs(T, K):
    return tuple(torch.full(s, float("nan"), device="cuda") for s in ((T,), (T,), (T, K)))


def both(inp):
    H, W, I, A, M = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask"))
    T, K = I.shape
    tau = inp["tau"]
    ws = torch.empty(kd.kd_topk_kl_workspace_size(T, H.shape[1], W.shape[1], K, H.dtype), dtype=torch.uint8,
                     device="cuda")
    a = outputs(T, K)
    kd.kd_topk_kl_fwd(H, W, I, A, M, tau, *a, ws)
    b = outputs(T, K)
    kd.kd_topk_kl_fwd_noalloc(H, W, I, A, M, tau, *b)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in a], [x.cpu().numpy() for x in b]


CASES = [
    # the output head, two forward chunks (4096 + 404 rows): the direct-to-LDS ring
    ("head T=4500 d=3072 V=128256 K=64 bf16", lambda: G.make_topk(
        4500, 3072, 128256, 64, torch.bfloat16, tau=1.3, mask="random10", number=50)),
    # smaller: ragged last vocabulary tile, still the ring
    ("T=700 d=384 V=2568 K=24 bf16", lambda: G.make_topk(
        700, 384, 2568, 24, torch.bfloat16, tau=0.8, mask="random10", number=51)),
    # smaller again, fp32: the register-staged mainloop
    ("T=300 d=136 V=1032 K=7 fp32", lambda: G.make_topk(
        300, 136, 1032, 7, torch.float32, tau=1.7, mask="random10", number=52)),
]


def test_noalloc_forward_matches_the_workspace_forward_on_calls_in_a_row():
    free0 = None
    for i, (name, make) in enumerate(CASES):
        inp = make()
        say(f"no-alloc forward, call {i + 1}: {name}")
        (kl_a, lse_a, z_a), (kl_b, lse_b, z_b) = both(inp)
        for what, x, y in (("kl", kl_a, kl_b), ("lse", lse_a, lse_b), ("z_topk", z_a, z_b)):
            assert np.all(np.isfinite(y)), f"{name}: {what} not fully written"
            np.testing.assert_array_equal(y, x, err_msg=f"{name}: {what}")
        m = inp["mask"].numpy() == 0
        assert np.all(kl_b[m] == 0) and np.all(z_b[m] == 0)
        # after the first call the array's address is known: later calls take
        # no device memory (torch's outputs and workspace above are freed and
        # reused by its caching allocator, which this does not see)
        free = torch.cuda.mem_get_info()[0]
        if free0 is not None:
            assert free >= free0 - (4 << 20), (free0, free)
        free0 = free if free0 is None else free0


def test_noalloc_forward_refuses_a_shape_beyond_its_scratch():
    T, d, V, K = 60000, 3072, 128256, 64
    H = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    W = torch.empty(d, V, dtype=torch.bfloat16, device="cuda")
    I = torch.zeros(T, K, dtype=torch.int32, device="cuda")
    A = torch.zeros(T, K, device="cuda")
    kl, lse = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    say("no-alloc forward above its scratch: refused on the host")
    with pytest.raises(kd.KDError, match="KD_NOALLOC_SCRATCH_BYTES"):
        kd.kd_topk_kl_fwd_noalloc(H, W, I, A, None, 1.0, kl, lse, None)
