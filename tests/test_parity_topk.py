"""GPU parity of the top-K loss: the HIP path (through the C-ABI binding)
against the fp64 oracle on the same seeded inputs, element by element.

Sizes span several 256-wide tiles and ragged tails in rows and vocabulary; the
full 3072 x 128256 head is checked on a 512-row slice (all outputs) and at
T = 4096 / 32768 on sampled rows (kl, lse, dH depend only on their row and W).
"""
import numpy as np
import pytest
import torch

import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, run_topk, say

pytestmark = pytest.mark.gpu


def oracle_all(inp):
    kl, lse, z = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"])
    dH, dW = O.topk_kl_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"])
    return dict(kl=kl, lse=lse, z=z, dH=dH, dW=dW)


def valid_of(inp):
    T = inp["H"].shape[0]
    return np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0


def check_all(got, want, inp, dtype, z_rtol=None):
    v = valid_of(inp)
    assert_kl(got["kl"], want["kl"], dtype, v)
    assert_lse(got["lse"], want["lse"], dtype, v)
    assert np.all(got["kl"][~v] == 0) and np.all(got["lse"][~v] == 0)
    if got["z"] is not None:
        assert np.all(got["z"][~v] == 0)
        np.testing.assert_allclose(got["z"][v], want["z"][v], rtol=z_rtol or 1e-5, atol=1e-5)
    assert np.all(got["dH"][~v] == 0)
    assert_grad(got["dH"], want["dH"], dtype, "dH")
    assert_grad(got["dW"], want["dW"], dtype, "dW")


# ---------------------------------------------------------------- the tiny fp32 workload
@pytest.mark.parametrize("g", ["mean", "normal"])
def test_tiny_fp32_workload(g):
    p = G.PRESETS["tiny_topk_fp32"]
    inp = G.make_preset(p, g=g)
    say(f"tiny_topk_fp32 T=256 d=256 V=4096 K=16 g={g}")
    got = run_topk(inp)
    check_all(got, oracle_all(inp), inp, torch.float32)


# ---------------------------------------------------------------- direct-load path, several backward chunks
# bf16 with d a multiple of 128 and V >= 256 takes the direct-load tile kernels:
# d % 256 = 128 gives a dW row block that is shifted up (its first rows are
# the previous block's and must not be added twice), V % 256 != 0 a last
# vocabulary tile shifted left, V % 128 != 0 the general dH mainloop, and a
# chunk smaller than T makes later chunks add to dW in place.
@pytest.mark.parametrize("T,d,V,K,tau,mask,chunk", [
    (700, 384, 1280, 16, 1.0, "none", 256),        # 3 chunks (256, 256, 188), dH on the direct-load path
    (900, 640, 2568, 24, 1.7, "random10", 512),    # partial last vocab tile, V % 128 = 8, masked rows
    (520, 256, 1024, 1, 1.0, "none", 256),         # K = 1, one row block, whole tiles only
])
def test_direct_load_path_chunks(T, d, V, K, tau, mask, chunk):
    inp = G.make_topk(T, d, V, K, torch.bfloat16, tau=tau, mask=mask, number=12, g="normal")
    say(f"direct-load T={T} d={d} V={V} K={K} chunk={chunk}")
    got = run_topk(inp, chunk_rows=chunk)
    check_all(got, oracle_all(inp), inp, torch.bfloat16, z_rtol=1e-4)


def test_chunk_size_does_not_change_the_result():
    # the chunked backward is a fixed-order split over tokens: any chunk size
    # gives the oracle's gradients (to rounding), and the forward is untouched
    inp = G.make_topk(1100, 384, 1536, 12, torch.bfloat16, tau=1.0, number=13, g="normal")
    say("chunk sizes 256 / 512 / 4096 on T=1100 d=384 V=1536")
    want = oracle_all(inp)
    runs = [run_topk(inp, want_z=False, chunk_rows=c) for c in (256, 512, 4096)]
    for r in runs:
        assert_grad(r["dH"], want["dH"], torch.bfloat16, "dH")
        assert_grad(r["dW"], want["dW"], torch.bfloat16, "dW")
        np.testing.assert_array_equal(r["kl"], runs[0]["kl"])


def test_runs_are_bitwise_deterministic():
    inp = G.make_topk(800, 384, 2568, 16, torch.bfloat16, tau=1.3, mask="random10", number=14, g="normal")
    say("determinism T=800 d=384 V=2568, two runs")
    a, b = run_topk(inp, chunk_rows=256), run_topk(inp, chunk_rows=256)
    for k in ("kl", "lse", "z", "dH", "dW"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


# ---------------------------------------------------------------- ragged shapes, both dtypes
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,d,V,K,tau,mask", [
    (300, 136, 1032, 7, 1.0, "none"),       # ragged rows (300 = 256 + 44), ragged vocab (4 tiles + 8)
    (513, 64, 520, 33, 0.7, "random10"),    # K > 32, two ragged edges, masked rows
    (37, 8, 264, 1, 2.5, "none"),           # K = 1 (cross-entropy), d = one chunk
    (1, 200, 2056, 5, 1.3, "none"),         # a single row
])
def test_ragged_shapes(dtype, T, d, V, K, tau, mask):
    inp = G.make_topk(T, d, V, K, dtype, tau=tau, mask=mask, number=11, g="normal")
    say(f"ragged T={T} d={d} V={V} K={K} tau={tau} {dtype}")
    got = run_topk(inp)
    check_all(got, oracle_all(inp), inp, dtype, z_rtol=1e-5 if dtype == torch.float32 else 1e-4)


def test_k_equals_v_and_duplicates():
    # K = V (a permutation per row), and a row set with duplicated indices
    inp = G.make_topk(70, 32, 64, 64, torch.float32, tau=1.0, number=12, g="normal")
    say("K=V=64 fp32")
    check_all(run_topk(inp), oracle_all(inp), inp, torch.float32)
    inp = G.make_topk(70, 32, 264, 12, torch.float32, tau=1.2, number=13, g="normal")
    I = inp["I"].clone()
    I[:, 3] = I[:, 0]
    I[::2, 7] = I[::2, 0]
    inp["I"] = I
    say("duplicate indices fp32")
    check_all(run_topk(inp), oracle_all(inp), inp, torch.float32)


# ---------------------------------------------------------------- exact gather (integer inputs)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gather_is_exact_on_integer_inputs(dtype):
    # H in {-2..2} and W in {-2..2}/8: every product and partial sum is exact in
    # fp32 accumulation, so the gathered logits must equal the oracle's bit for bit
    rng = np.random.default_rng(5)
    T, d, V, K = 300, 96, 1040, 20
    H = torch.from_numpy(rng.integers(-2, 3, (T, d)).astype(np.float32)).to(dtype)
    W = torch.from_numpy((rng.integers(-2, 3, (d, V)) / 8).astype(np.float32)).to(dtype)
    inp = dict(H=H, W=W, I=G.distinct_indices(7, T, K, V), A=G.teacher_logits(8, T, K, 3.0),
               mask=G.mask_random_rows(9, T, 30), g=torch.ones(T), tau=1.0)
    say(f"integer gather {dtype}")
    got = run_topk(inp)
    _, _, z = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], 1.0)
    np.testing.assert_array_equal(got["z"], z)


# ---------------------------------------------------------------- KL = 0
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_student_equal_to_teacher_gives_zero(dtype):
    # d = V = K = 16, W = identity, H_t[I_tk] = A_tk: s at the cached indices is
    # the teacher's own logits, so KL = 0 and the gradients vanish
    rng = np.random.default_rng(6)
    T, V = 300, 16
    A = torch.from_numpy(-np.sort(-rng.standard_normal((T, V)).astype(np.float32), axis=1)).to(dtype).float()
    I = torch.from_numpy(np.stack([rng.permutation(V) for _ in range(T)]).astype(np.int32))
    H = torch.zeros(T, V, dtype=torch.float32)
    H.scatter_(1, I.long(), A)
    inp = dict(H=H.to(dtype), W=torch.eye(V, dtype=dtype), I=I, A=A, mask=None, g=torch.ones(T), tau=1.0)
    say(f"KL=0 {dtype}")
    got = run_topk(inp)
    # prep's teacher log Z (natural base) and the tile epilogue's student log Z
    # (base 2) are two fp32 evaluations of the same number
    assert np.abs(got["kl"]).max() < 1e-5
    assert np.abs(got["dH"]).max() < 1e-5 and np.abs(got["dW"]).max() < 1e-3


# ---------------------------------------------------------------- masks and NaN
def test_masked_rows_exact_zero_and_nan_does_not_leak():
    inp = G.make_topk(400, 64, 520, 8, torch.bfloat16, tau=1.0, mask="random10", number=14, g="normal")
    m = inp["mask"].numpy() == 0
    clean = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    dirty = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in inp.items()}
    dirty["H"][torch.from_numpy(m)] = float("nan")
    dirty["A"][torch.from_numpy(m)] = float("nan")
    dirty["I"][torch.from_numpy(m)] = 10**9
    dirty["g"][torch.from_numpy(m)] = float("nan")
    say("masked rows with NaN")
    a, b = run_topk(clean), run_topk(dirty)
    for k in ("kl", "lse", "z", "dH", "dW"):
        assert np.all(np.isfinite(b[k])), k
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert np.all(b["kl"][m] == 0) and np.all(b["dH"][m] == 0)


def test_all_rows_masked():
    inp = G.make_topk(300, 64, 520, 8, torch.bfloat16, mask="random10", number=15, n_masked=300)
    say("all rows masked")
    got = run_topk(inp)
    for k in ("kl", "lse", "z", "dH", "dW"):
        assert not np.any(got[k]), k


# ---------------------------------------------------------------- the output head, 512-row slice
def test_head_slice_512_rows_all_outputs():
    p = G.PRESETS["head_topk_t4096"]
    inp = G.make_topk(512, p.d, p.V, p.K, p.dtype, tau=p.tau, number=p.number, g="normal")
    say("head slice T=512 d=3072 V=128256 K=64 bf16")
    got = run_topk(inp)
    check_all(got, oracle_all(inp), inp, torch.bfloat16, z_rtol=1e-4)


def test_head_slice_tau2_masked():
    inp = G.make_topk(300, 3072, 128256, 64, torch.bfloat16, tau=2.0, mask="random10", number=16, g="normal")
    say("head slice T=300 tau=2 masked bf16")
    got = run_topk(inp)
    check_all(got, oracle_all(inp), inp, torch.bfloat16, z_rtol=1e-4)


# ---------------------------------------------------------------- full sizes, sampled rows
def sample_rows(T, mask, n=256, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows |= {0, T - 1, 255, 256, 4095 % T, 4096 % T} | set(extra)
    if mask is not None:
        masked = np.nonzero(mask.numpy() == 0)[0]
        rows |= set(masked[:8].tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))


def check_sampled(got, inp, rows, dtype):
    kl, lse, z, dH = O.topk_kl_rows(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], rows)
    v = valid_of(inp)[rows]
    assert_kl(got["kl"][rows], kl, dtype, v)
    assert_lse(got["lse"][rows], lse, dtype, v)
    assert np.all(got["kl"][rows][~v] == 0)
    np.testing.assert_allclose(got["z"][rows][v], z[v], rtol=1e-4, atol=1e-5)
    assert_grad(got["dH"][rows], dH, dtype, "dH rows")
    # each sampled row's own dH within tolerance, not just the block
    for i in np.nonzero(v)[0]:
        assert_grad(got["dH"][rows[i]], dH[i], dtype, f"dH row {rows[i]}")


def test_head_t4096_sampled_rows():
    p = G.PRESETS["head_topk_t4096"]
    inp = G.make_preset(p, g="normal")
    say("head T=4096 sampled rows")
    got = run_topk(inp)
    check_sampled(got, inp, sample_rows(4096, None, n=256), torch.bfloat16)
    assert np.all(np.isfinite(got["dW"]))


def test_head_t32768_packed_sampled_rows():
    p = G.PRESETS["head_topk_t32768_packed"]
    inp = G.make_preset(p, g="normal")
    say("head T=32768 packed tau=2 sampled rows")
    got = run_topk(inp)
    rows = sample_rows(32768, inp["mask"], n=256, extra=[4096 * k - 206 for k in range(1, 9)]
                       + [4096 * k - 205 for k in range(1, 9)] + [4096 * k for k in range(1, 8)])
    check_sampled(got, inp, rows, torch.bfloat16)
    m = inp["mask"].numpy() == 0
    assert np.all(got["kl"][m] == 0) and np.all(got["dH"][m] == 0)


def test_out_of_range_index_in_a_valid_row_is_left_out_of_the_gather():
    # documented behaviour: an index outside [0, V) in a valid row never matches a
    # vocabulary column, so its entry drops out of the cross term (its z_topk stays
    # 0) while its probability still counts in the teacher terms
    inp = G.make_topk(300, 64, 520, 8, torch.bfloat16, tau=1.3, number=17, g="normal")
    bad = {(3, 2): 520 + 5, (10, 5): -3, (299, 0): 1 << 20}
    I = inp["I"].clone()
    for (t, k), v in bad.items():
        I[t, k] = v
    say("out-of-range indices in valid rows")
    got = run_topk(dict(inp, I=I))
    # the oracle on the in-range indices (the bad ones moved to column 0), then the
    # cross term of the moved entries taken back out
    I0 = I.clone()
    for (t, k) in bad:
        I0[t, k] = 0
    kl, lse, z = O.topk_kl_forward(inp["H"], inp["W"], I0, inp["A"], None, inp["tau"])
    logp = O.teacher_log_probs(O.as_f64(inp["A"]), inp["tau"])
    for (t, k) in bad:
        kl[t] += np.exp(logp[t, k]) * z[t, k] / inp["tau"]
        z[t, k] = 0.0
    assert_kl(got["kl"], kl, torch.bfloat16)
    assert_lse(got["lse"], lse, torch.bfloat16)
    np.testing.assert_allclose(got["z"], z, rtol=1e-4, atol=1e-5)
    for (t, k) in bad:
        assert got["z"][t, k] == 0



def test_largest_direct_load_chunk_sampled_rows():
    # chunk_rows past the direct-load reach is capped at 16384 rows at V = 128256:
    # a chunk of 16384 rows (a 4.2 GB dZ buffer, so offsets past 2^31 in dH and
    # dW) and one of 616 whose dW is added to the first's in place
    p = G.PRESETS["head_topk_t4096"]
    T = 17000
    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=1.0, number=18, g="normal")
    say("head T=17000, chunk_rows=32768 (capped at 16384)")
    got = run_topk(inp, want_z=False, chunk_rows=32768)
    rng = np.random.default_rng(8)
    rows = np.array(sorted(set(rng.choice(T, 256, replace=False).tolist()) | {0, 8400, 16383, 16384, 16639, T - 1}))
    kl, lse, _, dH = O.topk_kl_rows(inp["H"], inp["W"], inp["I"], inp["A"], None, 1.0, inp["g"], rows)
    assert_kl(got["kl"][rows], kl, torch.bfloat16)
    assert_lse(got["lse"][rows], lse, torch.bfloat16)
    assert_grad(got["dH"][rows], dH, torch.bfloat16, "dH rows")
    # every row of dZ sums to zero (mass 1), so each row of dW (d x V) sums to
    # zero over V up to the bf16 rounding of dZ, about 2^-9 of its norm
    dW = got["dW"]
    assert np.all(np.isfinite(dW))
    assert np.all(np.abs(dW.sum(axis=1)) <= 2e-2 * np.linalg.norm(dW, axis=1))
    # 4096-row chunks give the same gradients up to the fp32 order of the sums
    # (dH's split over V and dW's sum over chunks both depend on the chunk)
    say("head T=17000, chunk_rows=4096")
    ref = run_topk(inp, want_z=False, chunk_rows=4096)
    np.testing.assert_array_equal(got["kl"], ref["kl"])
    assert np.linalg.norm(got["dH"] - ref["dH"]) <= 1e-3 * np.linalg.norm(ref["dH"])
    assert np.linalg.norm(got["dW"] - ref["dW"]) <= 1e-5 * np.linalg.norm(ref["dW"])
