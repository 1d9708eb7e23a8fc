"""GPU parity of the full-vocabulary loss (teacher logits recomputed through a
frozen teacher head) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, run_full, say

pytestmark = pytest.mark.gpu


def oracle_all(inp):
    kl, ls, lt = O.full_kl_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"])
    dH, dW = O.full_kl_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], inp["g"])
    return dict(kl=kl, lse_s=ls, lse_t=lt, dH=dH, dW=dW)


def check_all(got, want, inp, dtype):
    T = inp["H"].shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(got["kl"], want["kl"], dtype, v)
    assert_lse(got["lse_s"], want["lse_s"], dtype, v)
    assert_lse(got["lse_t"], want["lse_t"], dtype, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], want["dH"], dtype, "dH")
    assert_grad(got["dW"], want["dW"], dtype, "dWs")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,d,dt,V,tau,mask", [
    (300, 136, 72, 1032, 1.0, "none"),
    (513, 64, 128, 520, 0.8, "random10"),
    (1, 40, 24, 264, 2.0, "none"),
])
def test_ragged_shapes(dtype, T, d, dt, V, tau, mask):
    inp = G.make_full(T, d, dt, V, dtype, tau=tau, mask=mask, number=21, g="normal")
    say(f"full ragged T={T} d={d} dt={dt} V={V} {dtype}")
    check_all(run_full(inp), oracle_all(inp), inp, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_equal_heads_give_exact_zero(dtype):
    # teacher and student run the same instructions on the same data
    inp = G.make_full(300, 64, 64, 520, dtype, number=22, g="normal")
    inp["Ht"], inp["Wt"] = inp["H"].clone(), inp["Ws"].clone()
    say(f"full equal heads {dtype}")
    got = run_full(inp)
    assert np.all(got["kl"] == 0)
    assert np.all(got["dH"] == 0) and np.all(got["dW"] == 0)


def test_full_slice_at_head_width():
    inp = G.make_full(256, 3072, 4096, 128256, torch.bfloat16, number=5, g="normal")
    say("full slice T=256 d=3072 dt=4096 V=128256")
    check_all(run_full(inp), oracle_all(inp), inp, torch.bfloat16)


def test_full_t16384_sampled_rows():
    p = G.PRESETS["full_vocab_t16384"]
    inp = G.make_preset(p, g="normal")
    say("full T=16384 sampled rows")
    got = run_full(inp)
    rng = np.random.default_rng(1)
    rows = np.array(sorted(set(rng.choice(16384, 256, replace=False).tolist())
                           | {0, 255, 256, 4095, 4096, 8191, 8192, 12287, 12288, 16383}))
    kl, ls, lt, dH = O.full_kl_rows(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], None, p.tau, inp["g"], rows)
    assert_kl(got["kl"][rows], kl, torch.bfloat16)
    assert_lse(got["lse_s"][rows], ls, torch.bfloat16)
    assert_lse(got["lse_t"][rows], lt, torch.bfloat16)
    assert_grad(got["dH"][rows], dH, torch.bfloat16, "dH rows")
    assert np.all(np.isfinite(got["dW"]))



def test_full_largest_direct_load_chunk_sampled_rows():
    # chunk_rows past the direct-load reach is capped at 16384 rows at V = 128256:
    # a chunk of 16384 rows (offsets past 2^31 in dH and dW) and one of 616
    p = G.PRESETS["full_vocab_t16384"]
    T = 17000
    inp = G.make_full(T, p.d, p.dt_hidden, p.V, p.dtype, tau=1.0, number=19, g="normal")
    say("full T=17000, chunk_rows=32768 (capped at 16384)")
    got = run_full(inp, chunk_rows=32768)
    rng = np.random.default_rng(9)
    rows = np.array(sorted(set(rng.choice(T, 256, replace=False).tolist()) | {0, 8400, 16383, 16384, 16639, T - 1}))
    kl, ls, lt, dH = O.full_kl_rows(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], None, 1.0, inp["g"], rows)
    assert_kl(got["kl"][rows], kl, torch.bfloat16)
    assert_lse(got["lse_s"][rows], ls, torch.bfloat16)
    assert_lse(got["lse_t"][rows], lt, torch.bfloat16)
    assert_grad(got["dH"][rows], dH, torch.bfloat16, "dH rows")
    # q - p sums to zero over V in every row, so each row of dW (d x V) does too,
    # up to the bf16 rounding of dZ
    dW = got["dW"]
    assert np.all(np.isfinite(dW))
    assert np.all(np.abs(dW.sum(axis=1)) <= 2e-2 * np.linalg.norm(dW, axis=1))
    say("full T=17000, chunk_rows=4096")
    ref = run_full(inp, chunk_rows=4096)
    np.testing.assert_array_equal(got["kl"], ref["kl"])
    assert np.linalg.norm(got["dH"] - ref["dH"]) <= 1e-3 * np.linalg.norm(ref["dH"])
    assert np.linalg.norm(got["dW"] - ref["dW"]) <= 1e-5 * np.linalg.norm(ref["dW"])


@pytest.mark.parametrize("T,d,dt,V,tau,mask,chunk", [
    (700, 384, 256, 1288, 1.0, "none", 256),       # last vocabulary tile shifted back, ragged row tile
    (900, 256, 640, 2568, 1.6, "random10", 512),   # teacher wider than student, masked rows
    (520, 128, 128, 128, 0.9, "none", 256),        # one vocabulary tile
])
def test_direct_load_path_chunks(T, d, dt, V, tau, mask, chunk):
    # d and dt multiples of 128: the direct-to-LDS mainloop with one ring over
    # both heads; several backward chunks accumulate into dW
    inp = G.make_full(T, d, dt, V, torch.bfloat16, tau=tau, mask=mask, number=24, g="normal")
    say(f"full direct-load T={T} d={d} dt={dt} V={V} chunk={chunk}")
    check_all(run_full(inp, chunk_rows=chunk), oracle_all(inp), inp, torch.bfloat16)


def test_full_runs_are_bitwise_deterministic():
    inp = G.make_full(600, 256, 384, 2056, torch.bfloat16, mask="random10", number=25, g="normal")
    say("full determinism")
    a, b = run_full(inp, chunk_rows=256), run_full(inp, chunk_rows=256)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
