"""GPU parity of the top-K loss with the output head split by vocabulary
columns (kd_topk_kl_fwd_shard, kd_topk_kl_shard_combine, kd_topk_kl_bwd_shard).
On one GPU the ranks run one after another and the all-gather is a stack of
their records.  Checked against the fp64 oracle: each shard's records and
teacher terms (oracle shard terms), the combined kl and lse, the summed z_topk
and dH partials, and the dW slices (unsharded oracle); at the headline shape
(8 shards of 16,032 columns) on sampled rows and by properties that hold at
any size.
"""
import numpy as np
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from oracle import kd_oracle as O
from tests.gpu_util import assert_grad, assert_kl, assert_lse, dev, say
from tests.test_parity_options import oracle_kw, options

pytestmark = pytest.mark.gpu

LN2 = np.log(2.0)


def run_shards(inp, cuts, chunk_rows=0, backward=True):
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    tau, o = inp["tau"], options(inp)
    parts, recs = [], []
    for v0, v1 in zip(cuts[:-1], cuts[1:]):
        Wc = W[:, v0:v1].contiguous()
        rec, trow, z = kd.topk_kl_shard_forward(H, Wc, v0, I, A, M, tau, want_z_topk=True, **o)
        recs.append(rec)
        parts.append(dict(v0=v0, vs=v1 - v0, Wc=Wc, rec=rec, trow=trow, z=z))
    kl, lse = kd.topk_kl_shard_combine(recs, parts[0]["trow"], M)
    if backward:
        for p in parts:
            p["dH"], p["dW"] = kd.topk_kl_shard_backward(H, p["Wc"], p["v0"], I, A, M, tau, lse, g, chunk_rows, **o)
    torch.cuda.synchronize()
    return parts, kl, lse


def np64(x):
    return x.cpu().double().numpy()


def check_records(parts, inp, dtype, rows=None):
    """Each shard's record against the oracle's shard terms (on `rows` if given)."""
    kw = oracle_kw(inp)
    sel = (lambda x: x) if rows is None else (lambda x: None if x is None else x[rows])
    H, I, A, mask = (sel(inp[k]) for k in ("H", "I", "A", "mask"))
    kwr = {k: (sel(v) if k != "ce_weight" else v) for k, v in kw.items()}
    v = np.ones(H.shape[0], bool) if mask is None else mask.numpy() != 0
    for p in parts:
        Wc = inp["W"][:, p["v0"]:p["v0"] + p["vs"]]
        ls, cross, ent, mass = O.topk_shard_terms(H, Wc, p["v0"], I, A, mask, inp["tau"], **kwr)
        rec, trow = sel(np64(p["rec"])), sel(np64(p["trow"]))
        got_ls = LN2 * (rec[:, 0] + np.log2(np.where(v, rec[:, 1], 1.0)))
        assert_lse(got_ls, ls, dtype, v)
        # the cross term is a sum of K logits weighted by p: compare on the scale of
        # the row's logits (the lse's tolerance times the weights' sum)
        np.testing.assert_allclose(rec[v, 2], cross[v], rtol=1e-3, atol=2e-3 * np.abs(ls[v]).max())
        np.testing.assert_allclose(trow[v, 0], ent[v], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(trow[v, 1], mass[v], rtol=1e-5)
        assert np.all(rec[~v] == 0) and np.all(trow[~v] == 0)


def check_combined(parts, kl, lse, inp, dtype):
    kw = oracle_kw(inp)
    want_kl, want_lse, want_z = O.topk_loss_forward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"],
                                                    inp["tau"], **kw)
    dH, dW = O.topk_loss_backward(inp["H"], inp["W"], inp["I"], inp["A"], inp["mask"], inp["tau"], inp["g"], **kw)
    T = want_kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(np64(kl), want_kl, dtype, v)
    assert_lse(np64(lse), want_lse, dtype, v)
    z = sum(np64(p["z"]) for p in parts)
    np.testing.assert_allclose(z[v], want_z[v], rtol=1e-4 if dtype == torch.bfloat16 else 1e-5, atol=1e-5)
    got_dH = sum(np64(p["dH"]) for p in parts)
    got_dW = np.concatenate([np64(p["dW"]) for p in parts], axis=1)
    assert_grad(got_dH, dH, dtype, "sum of dH partials")
    assert_grad(got_dW, dW, dtype, "dW slices")
    for p in parts:
        assert_grad(np64(p["dW"]), dW[:, p["v0"]:p["v0"] + p["vs"]], dtype, f"dW of shard at {p['v0']}")
        assert p["dH"].dtype == torch.float32
        assert np.all(np64(p["dH"])[~v] == 0)
    for x in (kl, lse):
        assert np.all(np64(x)[~v] == 0)


CASES = [
    # dtype, T, d, V, K, cuts (shard boundaries), chunk_rows, mask
    (torch.bfloat16, 700, 384, 2568, 16, (0, 640, 1288, 1800, 2568), 256, "random10"),  # 4 uneven shards
    (torch.bfloat16, 300, 136, 1032, 40, (0, 8, 520, 1032), 0, "none"),  # an 8-column shard, K > its width
    (torch.float32, 260, 64, 520, 9, (0, 260, 520), 256, "random10"),  # fp32 matrix cores
]


@pytest.mark.parametrize("dtype,T,d,V,K,cuts,chunk,mask", CASES)
def test_shards_match_the_oracle(dtype, T, d, V, K, cuts, chunk, mask):
    inp = G.make_topk(T, d, V, K, dtype, tau=1.2, mask=mask, number=81, g="normal")
    say(f"vocab shards {cuts} T={T} d={d} V={V} K={K} {dtype}")
    parts, kl, lse = run_shards(inp, cuts, chunk)
    check_records(parts, inp, dtype)
    check_combined(parts, kl, lse, inp, dtype)


def test_shards_with_every_option():
    inp = G.make_topk(700, 384, 2568, 24, torch.bfloat16, tau=1.0, mask="random10", number=82, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.3, number=82)
    cuts = (0, 1288, 1800, 2568)
    say(f"vocab shards {cuts} with every option")
    parts, kl, lse = run_shards(inp, cuts, 256)
    check_records(parts, inp, torch.bfloat16)
    check_combined(parts, kl, lse, inp, torch.bfloat16)


def test_one_shard_is_the_unsharded_call():
    # a single shard holding the whole head: the same kl, lse, z and dW bits as
    # the plain calls, dH the same values before rounding to bf16
    inp = G.make_topk(700, 384, 2568, 16, torch.bfloat16, tau=0.9, mask="random10", number=83, g="normal")
    say("one shard = the plain calls")
    parts, kl, lse = run_shards(inp, (0, 2568), 256)
    H, W, I, A, M, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "mask", "g"))
    kl0, lse0, z0 = kd.topk_kl_forward(H, W, I, A, M, 0.9, want_z_topk=True)
    dH0, dW0 = kd.topk_kl_backward(H, W, I, A, M, 0.9, lse0, g, 256)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np64(lse), np64(lse0))
    np.testing.assert_allclose(np64(kl), np64(kl0), rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(np64(parts[0]["z"]), np64(z0))
    np.testing.assert_array_equal(np64(parts[0]["dW"]), np64(dW0))
    np.testing.assert_array_equal(np64(parts[0]["dH"].to(torch.bfloat16)), np64(dH0))


def test_headline_shape_eight_shards_sampled_rows():
    p = G.PRESETS["head_topk_t4096"]
    inp = G.make_preset(p, g="normal")
    V = p.V
    cuts = tuple(range(0, V + 1, V // 8))
    assert len(cuts) == 9 and cuts[-1] == V
    say(f"head T=4096 d=3072 V=128256 in 8 shards of {V // 8} columns")
    H, W, I, A, g = (dev(inp[k]) for k in ("H", "W", "I", "A", "g"))
    recs, parts = [], []
    for v0, v1 in zip(cuts[:-1], cuts[1:]):
        Wc = W[:, v0:v1].contiguous()
        rec, trow, z = kd.topk_kl_shard_forward(H, Wc, v0, I, A, None, p.tau, want_z_topk=True)
        recs.append(rec)
        parts.append(dict(v0=v0, vs=v1 - v0, Wc=Wc, rec=rec, trow=trow, z=z))
    kl, lse = kd.topk_kl_shard_combine(recs, parts[0]["trow"], None)
    rng = np.random.default_rng(9)
    rows = np.array(sorted(set(rng.choice(4096, 64, replace=False).tolist()) | {0, 255, 256, 4095}))
    rows_d = torch.as_tensor(rows, device="cuda")
    dH_rows = torch.zeros(rows.size, p.d, dtype=torch.float64, device="cuda")
    dW_rowsum = torch.zeros(p.d, dtype=torch.float64, device="cuda")
    dW_rowsq = torch.zeros(p.d, dtype=torch.float64, device="cuda")
    for q in parts:
        dH, dW = kd.topk_kl_shard_backward(H, q["Wc"], q["v0"], I, A, None, p.tau, lse, g, 0)
        dH_rows += dH.index_select(0, rows_d).double()
        dW_rowsum += dW.double().sum(dim=1)
        dW_rowsq += dW.double().square().sum(dim=1)
        assert bool(torch.isfinite(dW).all())
        del dH, dW
    torch.cuda.synchronize()
    want_kl, want_lse, want_z, want_dH = O.topk_kl_rows(inp["H"], inp["W"], inp["I"], inp["A"], None, p.tau,
                                                         inp["g"], rows)
    assert_kl(np64(kl)[rows], want_kl, torch.bfloat16)
    assert_lse(np64(lse)[rows], want_lse, torch.bfloat16)
    z = sum(np64(q["z"].index_select(0, rows_d)) for q in parts)
    np.testing.assert_allclose(z, want_z, rtol=1e-4, atol=1e-5)
    assert_grad(dH_rows.cpu().numpy(), want_dH, torch.bfloat16, "sum of dH partials, sampled rows")
    # two shards' records on the sampled rows against the oracle's shard terms
    check_records([parts[0], parts[5]], inp, torch.bfloat16, rows=rows)
    # every row of dZ sums to zero over the whole head (mass 1), so each row of
    # dW, made of the 8 slices, sums to zero up to dZ's bf16 rounding
    assert np.all(np.abs(dW_rowsum.cpu().numpy()) <= 2e-2 * np.sqrt(dW_rowsq.cpu().numpy()))


# ---------------------------------------------------------------- full vocabulary
def run_full_shards(inp, cuts, chunk_rows=0, backward=True):
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    tau, r = inp["tau"], inp.get("rev_weight", 0.0)
    tr = dev(inp.get("tau_rows"))
    parts = []
    for v0, v1 in zip(cuts[:-1], cuts[1:]):
        Wsc, Wtc = Ws[:, v0:v1].contiguous(), Wt[:, v0:v1].contiguous()
        rec = kd.full_kl_shard_forward(H, Wsc, Ht, Wtc, M, tau, tau_rows=tr)
        parts.append(dict(v0=v0, vs=v1 - v0, Wsc=Wsc, Wtc=Wtc, rec=rec))
    kl, ls, lt, krev = kd.full_kl_shard_combine([p["rec"] for p in parts], M, r, want_kl_rev=True)
    if backward:
        for p in parts:
            p["dH"], p["dW"] = kd.full_kl_shard_backward(H, p["Wsc"], Ht, p["Wtc"], M, tau, ls, lt, g, chunk_rows,
                                                         tau_rows=tr, rev_weight=r, kl_rev=krev)
    torch.cuda.synchronize()
    return parts, dict(kl=kl, lse_s=ls, lse_t=lt, kl_rev=krev)


def full_kw(inp):
    return dict(tau_rows=inp.get("tau_rows"), rev_weight=inp.get("rev_weight", 0.0))


def check_full_records(parts, inp, dtype, rows=None):
    sel = (lambda x: x) if rows is None else (lambda x: None if x is None else x[rows])
    H, Ht, mask, tr = sel(inp["H"]), sel(inp["Ht"]), sel(inp["mask"]), sel(inp.get("tau_rows"))
    v = np.ones(H.shape[0], bool) if mask is None else mask.numpy() != 0
    for p in parts:
        c = slice(p["v0"], p["v0"] + p["vs"])
        ls, lt, ef, er = O.full_shard_terms(H, inp["Ws"][:, c], Ht, inp["Wt"][:, c], mask, inp["tau"], tau_rows=tr)
        rec = sel(np64(p["rec"]))
        one = lambda x: np.where(v, x, 1.0)
        assert_lse(LN2 * (rec[:, 0] + np.log2(one(rec[:, 1]))), ls, dtype, v)
        assert_lse(LN2 * (rec[:, 2] + np.log2(one(rec[:, 3]))), lt, dtype, v)
        # expectations of logit differences under the shard's softmaxes: on the
        # scale of the logits
        scale = np.abs(np.concatenate([ls[v], lt[v]])).max()
        np.testing.assert_allclose(LN2 * rec[v, 4] / rec[v, 3], ef[v], rtol=1e-3, atol=2e-3 * scale)
        np.testing.assert_allclose(LN2 * rec[v, 5] / rec[v, 1], er[v], rtol=1e-3, atol=2e-3 * scale)
        assert np.all(rec[~v] == 0)


def check_full_combined(parts, got, inp, dtype):
    kw = full_kw(inp)
    kl, ls, lt, krev = O.full_loss_forward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], **kw)
    dH, dW = O.full_loss_backward(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], inp["mask"], inp["tau"], inp["g"], **kw)
    T = kl.shape[0]
    v = np.ones(T, bool) if inp["mask"] is None else inp["mask"].numpy() != 0
    assert_kl(np64(got["kl"]), kl, dtype, v)
    assert_lse(np64(got["lse_s"]), ls, dtype, v)
    assert_lse(np64(got["lse_t"]), lt, dtype, v)
    assert_kl(np64(got["kl_rev"]), krev, dtype, v)
    assert_grad(sum(np64(p["dH"]) for p in parts), dH, dtype, "sum of dH partials")
    assert_grad(np.concatenate([np64(p["dW"]) for p in parts], axis=1), dW, dtype, "dWs slices")
    for p in parts:
        assert p["dH"].dtype == torch.float32
        assert np.all(np64(p["dH"])[~v] == 0)
    for x in got.values():
        assert np.all(np64(x)[~v] == 0)


FULL_CASES = [
    # dtype, T, d, dt, V, cuts, chunk_rows, options
    (torch.bfloat16, 700, 384, 256, 2568, (0, 640, 1288, 1800, 2568), 256, {}),
    (torch.bfloat16, 700, 384, 256, 2568, (0, 1288, 2568), 256, dict(tau_rows=True, rev_weight=0.3)),
    (torch.bfloat16, 300, 136, 72, 1032, (0, 8, 520, 1032), 0, dict(rev_weight=1.0)),
    (torch.float32, 260, 64, 128, 520, (0, 260, 520), 256, dict(tau_rows=True)),
]


@pytest.mark.parametrize("dtype,T,d,dt,V,cuts,chunk,opts", FULL_CASES)
def test_full_shards_match_the_oracle(dtype, T, d, dt, V, cuts, chunk, opts):
    inp = G.make_full(T, d, dt, V, dtype, tau=1.1, mask="random10", number=84, g="normal")
    if opts:
        inp = G.add_full_options(inp, number=84, **opts)
    say(f"full vocab shards {cuts} T={T} d={d} dt={dt} V={V} {dtype} {opts}")
    parts, got = run_full_shards(inp, cuts, chunk)
    check_full_records(parts, inp, dtype)
    check_full_combined(parts, got, inp, dtype)


def test_full_one_shard_is_the_unsharded_call():
    inp = G.make_full(700, 384, 256, 2568, torch.bfloat16, tau=0.9, mask="random10", number=85, g="normal")
    say("full vocab: one shard = the plain calls")
    parts, got = run_full_shards(inp, (0, 2568), 256)
    H, Ws, Ht, Wt, M, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "mask", "g"))
    kl0, ls0, lt0 = kd.full_kl_forward(H, Ws, Ht, Wt, M, 0.9)
    dH0, dW0 = kd.full_kl_backward(H, Ws, Ht, Wt, M, 0.9, ls0, lt0, g, 256)
    torch.cuda.synchronize()
    for a, b in ((got["kl"], kl0), (got["lse_s"], ls0), (got["lse_t"], lt0), (parts[0]["dW"], dW0)):
        np.testing.assert_array_equal(np64(a), np64(b))
    np.testing.assert_array_equal(np64(parts[0]["dH"].to(torch.bfloat16)), np64(dH0))


def test_full_t16384_eight_shards_sampled_rows():
    p = G.PRESETS["full_vocab_t16384"]
    inp = G.make_preset(p, g="normal")
    V = p.V
    cuts = tuple(range(0, V + 1, V // 8))
    say(f"full vocab T=16384 in 8 shards of {V // 8} columns")
    H, Ws, Ht, Wt, g = (dev(inp[k]) for k in ("H", "Ws", "Ht", "Wt", "g"))
    parts = []
    for v0, v1 in zip(cuts[:-1], cuts[1:]):
        Wsc, Wtc = Ws[:, v0:v1].contiguous(), Wt[:, v0:v1].contiguous()
        parts.append(dict(v0=v0, vs=v1 - v0, Wsc=Wsc, Wtc=Wtc, rec=kd.full_kl_shard_forward(H, Wsc, Ht, Wtc, None,
                                                                                             p.tau)))
    kl, ls, lt, _ = kd.full_kl_shard_combine([q["rec"] for q in parts], None)
    rng = np.random.default_rng(10)
    rows = np.array(sorted(set(rng.choice(p.T, 48, replace=False).tolist()) | {0, 4095, 4096, p.T - 1}))
    rows_d = torch.as_tensor(rows, device="cuda")
    dH_rows = torch.zeros(rows.size, p.d, dtype=torch.float64, device="cuda")
    dW_rowsum = torch.zeros(p.d, dtype=torch.float64, device="cuda")
    dW_rowsq = torch.zeros(p.d, dtype=torch.float64, device="cuda")
    for q in parts:
        dH, dW = kd.full_kl_shard_backward(H, q["Wsc"], Ht, q["Wtc"], None, p.tau, ls, lt, g, 0)
        dH_rows += dH.index_select(0, rows_d).double()
        dW_rowsum += dW.double().sum(dim=1)
        dW_rowsq += dW.double().square().sum(dim=1)
        assert bool(torch.isfinite(dW).all())
        del dH, dW
    torch.cuda.synchronize()
    want = O.full_loss_rows(inp["H"], inp["Ws"], inp["Ht"], inp["Wt"], None, p.tau, inp["g"], rows)
    assert_kl(np64(kl)[rows], want[0], torch.bfloat16)
    assert_lse(np64(ls)[rows], want[1], torch.bfloat16)
    assert_lse(np64(lt)[rows], want[2], torch.bfloat16)
    assert_grad(dH_rows.cpu().numpy(), want[4], torch.bfloat16, "sum of dH partials, sampled rows")
    check_full_records([parts[0], parts[7]], inp, torch.bfloat16, rows=rows)
    # rows of dZ sum to zero over the whole vocabulary, so do the rows of dWs
    assert np.all(np.abs(dW_rowsum.cpu().numpy()) <= 2e-2 * np.sqrt(dW_rowsq.cpu().numpy()))


@pytest.mark.parametrize("head", ["topk", "full"])
def test_shards_are_deterministic_and_follow_the_callers_stream(head):
    if head == "topk":
        inp = G.make_topk(700, 384, 2568, 16, torch.bfloat16, tau=1.1, mask="random10", number=86, g="normal")
    else:
        inp = G.make_full(700, 384, 256, 2568, torch.bfloat16, tau=1.1, mask="random10", number=87, g="normal")

    def run():
        if head == "topk":
            parts, kl, lse = run_shards(inp, (0, 1288, 2568), 256)
            outs = [kl, lse]
        else:
            parts, got = run_full_shards(inp, (0, 1288, 2568), 256)
            outs = list(got.values())
        return [np64(x) for x in outs] + [np64(p[k]) for p in parts for k in ("rec", "dH", "dW")]

    say(f"{head} shards: two runs, then on a second stream")
    a, b = run(), run()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        c = run()
    for i, (x, y, z) in enumerate(zip(a, b, c)):
        np.testing.assert_array_equal(x, y, err_msg=f"output {i}, second run")
        np.testing.assert_array_equal(x, z, err_msg=f"output {i}, second stream")


@pytest.mark.parametrize("head", ["topk", "full"])
def test_shards_with_every_row_masked(head):
    say(f"{head} shards, every row masked")
    if head == "topk":
        inp = G.make_topk(300, 256, 1288, 8, torch.bfloat16, mask="random10", n_masked=300, number=88, g="normal")
        parts, kl, lse = run_shards(inp, (0, 640, 1288), 256)
        outs = [kl, lse]
    else:
        inp = G.make_full(300, 256, 128, 1288, torch.bfloat16, mask="random10", n_masked=300, number=89, g="normal")
        parts, got = run_full_shards(inp, (0, 640, 1288), 256)
        outs = list(got.values())
    assert int(inp["mask"].sum()) == 0
    for x in outs + [p[k] for p in parts for k in ("rec", "dH", "dW")]:
        assert np.all(np64(x) == 0)
