"""GPU parity at the sizes only long contexts reach, and where the gather must
be exact on the path the output-head workload takes.

- The loss-only sweep's long points (T = 65,536 and 262,144; d = 3072,
  V = 128256, K = 64, bf16): 64 forward chunks, pair-array offsets near 2^24
  and 1.6 GB of H.  "Efficient Knowledge Distillation for LLMs: Offline Top-K
  Logits and a Fused Chunked KL Loss", §4 "Controlled loss-only benchmark"
  (peak memory up to 256K tokens) and §5 "Benchmark limitations" (the 4K-256K
  sweep).  kl, lse, z_topk and dH of a row depend only on that row and W, so
  they are checked against the oracle on a seeded sample of rows that takes in
  every row next to a 4096-row chunk boundary; dW is checked through a
  property that holds at any size (every dZ row sums to zero, so every dW row
  does, up to the bf16 rounding of dZ).
- An exact gather on the direct-to-LDS ring (bf16, d a multiple of 128, V at
  least one whole tile): integer-valued operands make every logit exact in
  fp32, so z_topk must equal the oracle bit for bit, in the two-call and the
  single-call forms (§3 "Offline distillation": only the K cached student
  logits are gathered).
- dW of several backward chunks against the oracle at the full head width, and
  the split of a packed long-context batch into halves whose dW add up to the
  whole's (§3 "Fused chunked KL": the backward runs chunk by chunk).
"""
import numpy as np
import pytest
import torch

import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, rel_fro, run_topk, run_topk_sampled, say

import chunked_kl_loss_logit_amd as kd

pytestmark = pytest.mark.gpu


def boundary_rows(T, n=256, seed=0):
    """n seeded rows plus the first and last row and the rows on either side of
    every 4096-row chunk boundary."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    for b in range(4096, T, 4096):
        rows |= {b - 1, b, b + 1}
    return np.array(sorted(r for r in rows if 0 <= r < T))


@pytest.mark.parametrize("T", [65536, 262144])
def test_sweep_long_context_sampled_rows(T):
    p = G.sweep_preset(T)
    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=p.tau, teacher_var=p.teacher_var, number=p.number, g="normal")
    rows = boundary_rows(T, seed=T)
    assert rows.size >= 256 + 2 * (T // 4096)
    say(f"sweep T={T} d=3072 V=128256 K=64 bf16, {rows.size} sampled rows")
    got = run_topk_sampled(inp, rows)
    kl, lse, z, dH = O.topk_kl_rows(inp["H"], inp["W"], inp["I"], inp["A"], None, p.tau, inp["g"], rows)
    assert_kl(got["kl"], kl, torch.bfloat16)
    assert_lse(got["lse"], lse, torch.bfloat16)
    np.testing.assert_allclose(got["z"], z, rtol=1e-4, atol=1e-5)
    assert_grad(got["dH"], dH, torch.bfloat16, "dH rows")
    for i, r in enumerate(rows):
        assert_grad(got["dH"][i], dH[i], torch.bfloat16, f"dH row {r}")
    assert got["dW_finite"]
    assert np.all(np.abs(got["dW_rowsum"]) <= 2e-2 * got["dW_rownorm"])
    assert np.all(got["dW_rownorm"] > 0)


# ---------------------------------------------------------------- exact gather on the direct-to-LDS ring
def integer_inputs(T, d, V, K, seed):
    # H in {-2..2} and W in {-2..2}/8 are exact in bf16, and every partial sum
    # of their products is a multiple of 1/8 below 2^21: exact in fp32
    rng = np.random.default_rng(seed)
    H = torch.from_numpy(rng.integers(-2, 3, (T, d)).astype(np.float32)).to(torch.bfloat16)
    W = torch.from_numpy((rng.integers(-2, 3, (d, V)) / 8).astype(np.float32)).to(torch.bfloat16)
    return dict(H=H, W=W, I=G.distinct_indices(seed + 1, T, K, V), A=G.teacher_logits(seed + 2, T, K, 3.0),
                mask=G.mask_random_rows(seed + 3, T, T // 10), g=G.normal(seed + 4, (T,), 1.0, torch.float32),
                tau=1.0)


@pytest.mark.parametrize("d,V,K", [(128, 1280, 64), (384, 2568, 24)])
def test_gather_is_exact_on_the_direct_load_ring(d, V, K):
    # T = 4500: two forward chunks (4096 + 404 rows) and, at chunk_rows = 1024,
    # five backward chunks; V = 2568 ends on a vocabulary tile shifted left
    T = 4500
    inp = integer_inputs(T, d, V, K, seed=40 + d)
    _, _, want = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], 1.0)
    m = inp["mask"].numpy() == 0
    say(f"exact gather on the ring, two calls: T={T} d={d} V={V} K={K}")
    got = run_topk(inp, chunk_rows=1024)
    np.testing.assert_array_equal(got["z"], want)
    assert np.all(got["z"][m] == 0)
    say(f"exact gather on the ring, single call: T={T} d={d} V={V} K={K}")
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    _, _, z1, _, _ = kd.topk_kl_forward_backward(H, W, I, A, M, 1.0, g, chunk_rows=1024, want_z_topk=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z1.cpu().double().numpy(), want)


# ---------------------------------------------------------------- dW over several chunks, full head width
def test_full_width_dw_over_four_chunks_matches_the_oracle():
    p = G.PRESETS["head_topk_t4096"]
    T = 1024
    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=1.3, mask="random10", number=41, g="normal")
    say("head width T=1024 (102 masked), chunk_rows=256: four backward chunks")
    got = run_topk(inp, want_z=False, chunk_rows=256)
    kl, lse, _ = O.topk_kl_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"])
    dH, dW = O.topk_kl_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"],
                                row_block=256)
    v = inp["mask"].numpy() != 0
    assert_kl(got["kl"], kl, torch.bfloat16, v)
    assert_lse(got["lse"], lse, torch.bfloat16, v)
    assert_grad(got["dH"], dH, torch.bfloat16, "dH")
    assert_grad(got["dW"], dW, torch.bfloat16, "dW")


def test_packed_long_context_halves_add_up():
    # dW(T) = dW(first half) + dW(second half) on the packed long-context
    # workload (tau 2, 205 padding rows per 4096-row sequence): eight chunks
    # against two runs of four.  The halves compact their rows on their own, so
    # their chunks hold other rows than the whole's: equal only to rounding.
    p = G.PRESETS["head_topk_t32768_packed"]
    inp = G.make_preset(p, g="normal")
    T = p.T
    halves = [{k: (v[s] if torch.is_tensor(v) and v.shape[0] == T else v) for k, v in inp.items()}
              for s in (slice(0, T // 2), slice(T // 2, T))]
    for h in halves:
        h["W"] = inp["W"]
    say("packed T=32768 tau=2: the whole")
    whole = run_topk(inp, want_z=False)
    say("packed T=32768 tau=2: the two halves")
    a, b = (run_topk(h, want_z=False) for h in halves)
    assert rel_fro(a["dW"] + b["dW"], whole["dW"]) <= 1e-4
    assert rel_fro(np.concatenate([a["dH"], b["dH"]]), whole["dH"]) <= 1e-4
    np.testing.assert_allclose(np.concatenate([a["kl"], b["kl"]]), whole["kl"], rtol=1e-5, atol=1e-6)
