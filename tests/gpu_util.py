"""Helpers of the GPU parity tests: run the HIP path through the C-ABI binding
on CPU-generated inputs and compare with the fp64 oracle."""
import sys

import numpy as np
import torch

import chunked_kl_loss_logit_amd as kd

# Tolerances (stated for the loss in the problem statement; per-token floor for
# near-zero KL derived from fp32 rounding of log Z, about 1e-6 relative):
#   bf16 inputs: per token |dKL| <= 1e-3 |KL| + 1e-4, loss sum rel 1e-3,
#                dH and dW rel-Frobenius 1e-2
#   fp32 inputs: every quantity rel 1e-5 (per token |dKL| <= 1e-5 |KL| + 1e-5)
TOL = {
    torch.bfloat16: dict(kl_rel=1e-3, kl_abs=1e-4, lse_rel=1e-4, grad=1e-2),
    torch.float32: dict(kl_rel=1e-5, kl_abs=1e-5, lse_rel=1e-6, grad=1e-5),
}


def say(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(x):
    return None if x is None else x.cuda().contiguous()


def run_topk(inp, want_z=True, chunk_rows=0):
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    tau = inp["tau"]
    kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, want_z_topk=want_z)
    dH, dW = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, chunk_rows)
    torch.cuda.synchronize()
    return dict(kl=kl.cpu().double().numpy(), lse=lse.cpu().double().numpy(),
                z=None if z is None else z.cpu().double().numpy(),
                dH=dH.cpu().double().numpy(), dW=dW.cpu().double().numpy())


def run_full(inp, chunk_rows=0):
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    tau = inp["tau"]
    kl, ls, lt = kd.full_kl_forward(H, Ws, Ht, Wt, M, tau)
    dH, dW = kd.full_kl_backward(H, Ws, Ht, Wt, M, tau, ls, lt, g, chunk_rows)
    torch.cuda.synchronize()
    return dict(kl=kl.cpu().double().numpy(), lse_s=ls.cpu().double().numpy(), lse_t=lt.cpu().double().numpy(),
                dH=dH.cpu().double().numpy(), dW=dW.cpu().double().numpy())


def rel_fro(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def assert_kl(got, want, dtype, valid=None):
    t = TOL[dtype]
    if valid is not None:
        got, want = got[valid], want[valid]
    err = np.abs(got - want)
    bound = t["kl_rel"] * np.abs(want) + t["kl_abs"]
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{bad.size} tokens off, worst {err.max():.3e} at {err.argmax()} (kl {want[err.argmax()]:.4f})"
    s_got, s_want = got.sum(), want.sum()
    assert abs(s_got - s_want) <= t["kl_rel"] * abs(s_want) + 1e-12, (s_got, s_want)


def assert_lse(got, want, dtype, valid=None):
    if valid is not None:
        got, want = got[valid], want[valid]
    np.testing.assert_allclose(got, want, rtol=TOL[dtype]["lse_rel"], atol=1e-5)


def assert_grad(got, want, dtype, what):
    r = rel_fro(got, want)
    assert r <= TOL[dtype]["grad"], f"{what}: rel Frobenius {r:.3e}"


def run_topk_sampled(inp, rows, chunk_rows=0, want_z=True):
    """The top-K forward + backward on the GPU at any T, copying back only the
    sampled rows' kl, lse, z_topk and dH, plus per-row statistics of dW
    (its row sums and norms, in float64) and whether all of dW is finite."""
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    tau = inp["tau"]
    kl, lse, z = kd.topk_kl_forward(H, W, I, A, M, tau, want_z_topk=want_z)
    dH, dW = kd.topk_kl_backward(H, W, I, A, M, tau, lse, g, chunk_rows)
    r = torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()
    out = dict(kl=kl[r].cpu().double().numpy(), lse=lse[r].cpu().double().numpy(),
               z=None if z is None else z[r].cpu().double().numpy(), dH=dH[r].cpu().double().numpy(),
               dW_rowsum=dW.double().sum(dim=1).cpu().numpy(), dW_rownorm=dW.double().norm(dim=1).cpu().numpy(),
               dW_finite=bool(torch.isfinite(dW).all().item()),
               kl_masked_zero=True if M is None else bool((kl[M == 0] == 0).all().item()),
               dH_masked_zero=True if M is None else bool((dH[M == 0] == 0).all().item()))
    torch.cuda.synchronize()
    del H, W, I, A, M, g, kl, lse, z, dH, dW
    torch.cuda.empty_cache()
    return out
