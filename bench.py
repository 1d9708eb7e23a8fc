"""Throughput of the fused chunked KL loss, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --sweep          # loss-only scaling sweep, one line per T
    python bench.py --copy-probe N   # plain copy of N bytes (counter calibration)
    python bench.py --workload head_topk_t4096_vshard8   # one rank of an 8-way vocabulary split
                                                         # (also full_vocab_t16384_vshard8)

A step of the top-K workloads is one kd_topk_kl_fwd plus one kd_topk_kl_bwd
over one batch of synthetic rows (inputs already in HBM): the output
projection, online log Z, top-K gather, per-token KL, and the chunked backward
(recomputed projection, dZ, dH, dW).  A step of the full-vocabulary workload
is kd_full_kl_fwd plus kd_full_kl_bwd (or, with --one-call, one
kd_full_kl_fwd_bwd).  The default run prints ONE JSON line for the
output-head workload (T=4096, d=3072, V=128256, K=64); the same workload
through the single-call kd_topk_kl_fwd_bwd (no recompute), the packed
long-context workload and the full-vocabulary workload (two calls and single
call) ride along in its "extra" object.

The loss-only benchmark of "Efficient Knowledge Distillation for LLMs: Offline
Top-K Logits and a Fused Chunked KL Loss" (App. B) times the same path: output
projection plus KL forward/backward, on deterministic synthetic inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused KL fwd+bwd tokens/s (d=3072,V=128256) + % bf16 MFMA peak; peak extra HBM"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
TILE_KERNELS = ("topk_fwd_tile", "topk_dz_tile", "full_fwd_tile", "full_dz_tile", "full_teacher_tile", "full_student_tile",
                "dh_tile", "dw_tile")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="head_topk_t4096")
    ap.add_argument("--T", type=int, default=0, help="override the row count")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extra", action="store_true", help="skip the packed and full-vocabulary workloads")
    ap.add_argument("--one-call", action="store_true",
                    help="full-vocabulary workload: time the single forward + backward call")
    ap.add_argument("--no-protocol", action="store_true",
                    help="skip the pages' 15-iteration protocol pass (short profiling runs)")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--sweep", action="store_true", help="T in 4096, 16384, 65536, 262144: one line each")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 4 times (calibrates HBM byte counters)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the vendor GEMM (torch.matmul) on the head's three contraction shapes")
    ap.add_argument("--operand-probe", choices=("seeded", "zero"), default=None,
                    help="only time the headline's two calls on its seeded operands or on all-zero H and W "
                         "(same shapes and instructions): a diagnostic of how the clock depends on the data, "
                         "not the metric")
    return ap.parse_args()


def copy_probe(nbytes: int):
    """A plain copy kernel of known size: reads and writes nbytes per launch.

    Its FETCH_SIZE / WRITE_SIZE counter readings give the factor that turns
    those counters into bytes for the loss kernels."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 4}))


def source_digest() -> str:
    """SHA-256 over the library's device and interface sources (names + bytes)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_kl_loss_logit_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)) + [os.path.join(ROOT, "include", "kdloss.h")]
    for p in files:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter table, or
    None when there is none for this workload or the sources changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("workload") != workload or data.get("source_digest") != source_digest():
        return None
    return data.get("kernels", {}).get(kernel, {}).get("bytes_per_launch")


def cpu_baseline(inp, rows: int):
    """The oracle, as it stands, on the first `rows` rows of the same workload."""
    from oracle import kd_oracle as O
    sl = {k: (v[:rows] if hasattr(v, "shape") and v.shape[0] == inp["H"].shape[0] else v) for k, v in inp.items()}
    W = O.as_f64(inp["W"])
    t0 = time.perf_counter()
    O.topk_kl_forward(sl["H"], W, sl["I"], sl["A"], sl["mask"], inp["tau"])
    O.topk_kl_backward(sl["H"], W, sl["I"], sl["A"], sl["mask"], inp["tau"], sl["g"])
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {rows} of {inp['H'].shape[0]} rows, forward + backward, fp64 NumPy "
                      f"(BLAS threads = cores), {dt:.1f} s"}


def timed(step, steps: int, warmup: int):
    """Warmup steps, then exactly `steps` timed steps with the library's
    per-launch profiling off (the timed region is the plain calls); then, in
    a pass of its own, the same number of steps with every launch bracketed
    by HIP events on its stream, for the per-kernel table.  Returns (ms per
    step, {kernel: (launches, total ms)}, steps of the kernel pass)."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kd.profile_reset()
    kd.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kd.profile_enable(False)
    return elapsed / steps * 1e3, kd.profile_read(), steps


def pages_protocol(step, iterations: int = 15, first: int = 10, last: int = 13):
    """The loss benchmark's own protocol ("Efficient Knowledge Distillation for
    LLMs ...", App. A "Profiling": 15-iteration runs, captured over iterations
    10-13): `iterations` steps each bracketed by HIP events on the current
    stream, and the mean step time of iterations first..last (1-based)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iterations)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    cap = ms[first - 1:last]
    return {"iterations": iterations, "captured": f"{first}-{last}", "ms_per_step": sum(cap) / len(cap),
            "ms_captured": [round(x, 4) for x in cap]}


def kernel_table(prof, steps: int):
    per_step = sum(tot for _, tot in prof.values()) / steps
    return {k: {"launches": n, "avg_ms": tot / n, "ms_per_step": tot / steps, "share": tot / steps / per_step}
            for k, (n, tot) in prof.items()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def dominant(prof, flops_per_step: dict, steps: int):
    """The tile kernel with the most GPU time in the kernel pass, and its
    achieved rate: algorithmic flops of one launch / its average launch
    duration (HIP events on the launch stream)."""
    dom = max((k for k in prof if k in TILE_KERNELS), key=lambda k: prof[k][1])
    n_l, tot_ms = prof[dom]
    per_launch = flops_per_step[dom] / (n_l / steps)
    return dom, per_launch / (tot_ms / n_l * 1e-3) / 1e12


def run_topk(p, T: int, steps: int, warmup: int, chunk_rows: int, protocol: bool = False):
    """Time the top-K loss on preset p at T rows (with protocol, also the
    pages' 15-iteration protocol in a pass of its own)."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=p.tau, teacher_var=p.teacher_var, mask=p.mask,
                      number=p.number, seq_len=p.seq_len, n_pad=p.n_pad, g="mean")
    dev = torch.device("cuda:0")
    H, W, I, A, g = (inp[k].to(dev) for k in ("H", "W", "I", "A", "g"))
    M = None if inp["mask"] is None else inp["mask"].to(dev)
    n_valid = T if inp["mask"] is None else int(inp["mask"].sum())
    d, V, K, tau = p.d, p.V, p.K, p.tau
    kl = torch.empty(T, device=dev)
    lse = torch.empty(T, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, device=dev)
    torch.cuda.synchronize()

    # peak extra HBM of one forward + backward: the workspace is the only
    # allocation the calls need (the library allocates nothing itself)
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws = torch.empty(kd.kd_topk_kl_workspace_size(T, d, V, K, p.dtype, chunk_rows), dtype=torch.uint8, device=dev)
    kd.kd_topk_kl_fwd(H, W, I, A, M, tau, kl, lse, None, ws)
    kd.kd_topk_kl_bwd(H, W, I, A, M, tau, lse, g, dH, dW, chunk_rows, ws)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base + lse.numel() * 4  # + saved lse

    def step():
        kd.kd_topk_kl_fwd(H, W, I, A, M, tau, kl, lse, None, ws)
        kd.kd_topk_kl_bwd(H, W, I, A, M, tau, lse, g, dH, dW, chunk_rows, ws)

    ms, prof, ksteps = timed(step, steps, warmup)
    # algorithmic flops per step of each tile kernel (valid rows only)
    fl = {k: 2.0 * n_valid * d * V for k in ("topk_fwd_tile", "topk_dz_tile", "dh_tile", "dw_tile")}
    dom, achieved = dominant(prof, fl, ksteps)
    out = {"workload": p.name, "T": T, "valid_rows": n_valid, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
           "valid_tokens_per_s": n_valid / (ms * 1e-3),
           "credited_tflops": 6.0 * n_valid * d * V / (ms * 1e-3) / 1e12,
           "peak_extra_hbm_bytes": int(peak_extra), "dominant": dom, "dominant_tflops": achieved,
           "kernels": kernel_table(prof, ksteps), "steps_timed": steps}
    out["mfma_frac_credited"] = out["credited_tflops"] / PEAK_BF16_TFLOPS
    out["mfma_frac_executed"] = out["mfma_frac_credited"] * 8.0 / 6.0  # the backward recomputes the projection
    if protocol:
        out["pages_protocol"] = pages_protocol(step)
    del H, W, I, A, g, M, kl, lse, dH, dW, ws
    torch.cuda.empty_cache()
    return out, inp


def run_topk_fused(p, T: int, steps: int, warmup: int, chunk_rows: int):
    """Time the single-call forward + backward (kd_topk_kl_fwd_bwd, no recompute) on preset p."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=p.tau, teacher_var=p.teacher_var, mask=p.mask,
                      number=p.number, seq_len=p.seq_len, n_pad=p.n_pad, g="mean")
    dev = torch.device("cuda:0")
    H, W, I, A, g = (inp[k].to(dev) for k in ("H", "W", "I", "A", "g"))
    M = None if inp["mask"] is None else inp["mask"].to(dev)
    n_valid = T if inp["mask"] is None else int(inp["mask"].sum())
    del inp
    d, V, K, tau = p.d, p.V, p.K, p.tau
    kl = torch.empty(T, device=dev)
    lse = torch.empty(T, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws = torch.empty(kd.kd_topk_kl_fwd_bwd_workspace_size(T, d, V, K, p.dtype, chunk_rows), dtype=torch.uint8,
                     device=dev)

    def step():
        kd.kd_topk_kl_fwd_bwd(H, W, I, A, M, tau, g, kl, lse, None, dH, dW, chunk_rows, ws)

    step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base
    ms, prof, ksteps = timed(step, steps, warmup)
    fl = {k: 2.0 * n_valid * d * V for k in ("topk_fwd_tile", "dh_tile", "dw_tile")}
    dom, achieved = dominant(prof, fl, ksteps)
    cred = 6.0 * n_valid * d * V / (ms * 1e-3) / 1e12
    out = {"workload": p.name + "_one_call", "T": T, "valid_rows": n_valid, "ms_per_step": ms,
           "tokens_per_s": T / (ms * 1e-3), "valid_tokens_per_s": n_valid / (ms * 1e-3), "credited_tflops": cred,
           "mfma_frac_credited": cred / PEAK_BF16_TFLOPS, "mfma_frac_executed": cred / PEAK_BF16_TFLOPS,
           "peak_extra_hbm_bytes": int(peak_extra), "dominant": dom, "dominant_tflops": achieved,
           "kernels": kernel_table(prof, ksteps), "steps_timed": steps}
    del H, W, I, A, g, M, kl, lse, dH, dW, ws
    torch.cuda.empty_cache()
    return out


def run_full(p, steps: int, warmup: int, chunk_rows: int, one_call: bool = False):
    """Time the full-vocabulary loss on preset p: the forward and backward
    calls, or with one_call the single call that keeps both heads' logits of
    a chunk instead of recomputing them (kd_full_kl_fwd_bwd)."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    T, d, dt, V, tau = p.T, p.d, p.dt_hidden, p.V, p.tau
    inp = G.make_full(T, d, dt, V, p.dtype, tau=tau, number=p.number, g="mean")
    dev = torch.device("cuda:0")
    H, Ws, Ht, Wt, g = (inp[k].to(dev) for k in ("H", "Ws", "Ht", "Wt", "g"))
    del inp
    kl = torch.empty(T, device=dev)
    ls = torch.empty(T, device=dev)
    lt = torch.empty(T, device=dev)
    dH = torch.empty_like(H)
    dW = torch.empty(d, V, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    if one_call:
        ws = torch.empty(kd.kd_full_kl_fwd_bwd_workspace_size(T, d, dt, V, p.dtype, chunk_rows), dtype=torch.uint8,
                         device=dev)

        def step():
            kd.kd_full_kl_fwd_bwd(H, Ws, Ht, Wt, None, tau, g, kl, ls, lt, dH, dW, chunk_rows, ws)
    else:
        ws = torch.empty(kd.kd_full_kl_workspace_size(T, d, dt, V, p.dtype, chunk_rows), dtype=torch.uint8,
                         device=dev)

        def step():
            kd.kd_full_kl_fwd(H, Ws, Ht, Wt, None, tau, kl, ls, lt, ws)
            kd.kd_full_kl_bwd(H, Ws, Ht, Wt, None, tau, ls, lt, g, dH, dW, chunk_rows, ws)

    step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base + (0 if one_call else 2 * T * 4)  # + saved lse_s, lse_t
    ms, prof, ksteps = timed(step, steps, warmup)
    fl = {"full_fwd_tile": 2.0 * T * (d + dt) * V, "full_dz_tile": 2.0 * T * (d + dt) * V,
          "full_teacher_tile": 2.0 * T * dt * V, "full_student_tile": 2.0 * T * d * V,
          "dh_tile": 2.0 * T * d * V, "dw_tile": 2.0 * T * d * V}
    dom, achieved = dominant(prof, fl, ksteps)
    credited = (2.0 * (d + dt) + 4.0 * d) * V * T
    executed = ((2.0 if one_call else 4.0) * (d + dt) + 4.0 * d) * V * T
    out = {"workload": p.name + ("_one_call" if one_call else ""), "T": T, "ms_per_step": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "credited_tflops": credited / (ms * 1e-3) / 1e12,
           "mfma_frac_credited": credited / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "mfma_frac_executed": executed / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "peak_extra_hbm_bytes": int(peak_extra), "dominant": dom, "dominant_tflops": achieved,
           "kernels": kernel_table(prof, ksteps), "steps_timed": steps}
    del H, Ws, Ht, Wt, g, kl, ls, lt, dH, dW, ws
    torch.cuda.empty_cache()
    return out


def run_topk_shard(p, T: int, R: int, steps: int, warmup: int, chunk_rows: int):
    """Time one rank's step of the top-K loss with the head split by vocabulary
    over R ranks (rank 0: columns [0, V/R)): its forward, the combine of R
    records and its backward.  The other ranks' records are copies of its own,
    made once before timing (the exchange between GPUs is not part of one
    GPU's work; the combine does the same arithmetic on any records)."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    inp = G.make_topk(T, p.d, p.V, p.K, p.dtype, tau=p.tau, teacher_var=p.teacher_var, mask=p.mask,
                      number=p.number, seq_len=p.seq_len, n_pad=p.n_pad, g="mean")
    dev = torch.device("cuda:0")
    Vs = p.V // R
    H, I, A, g = (inp[k].to(dev) for k in ("H", "I", "A", "g"))
    W = inp["W"][:, :Vs].contiguous().to(dev)
    M = None if inp["mask"] is None else inp["mask"].to(dev)
    n_valid = T if inp["mask"] is None else int(inp["mask"].sum())
    del inp
    d, K, tau = p.d, p.K, p.tau
    rec = torch.empty(R, T, 4, device=dev)
    trow = torch.empty(T, 2, device=dev)
    kl = torch.empty(T, device=dev)
    lse = torch.empty(T, device=dev)
    dH = torch.empty(T, d, device=dev)
    dW = torch.empty(d, Vs, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws = torch.empty(kd.kd_topk_kl_shard_workspace_size(T, d, Vs, 0, K, p.dtype, chunk_rows), dtype=torch.uint8,
                     device=dev)

    def step():
        kd.kd_topk_kl_fwd_shard(H, W, 0, I, A, M, tau, None, rec[0], trow, None, ws)
        kd.kd_topk_kl_shard_combine(rec, trow, M, kl, lse)
        kd.kd_topk_kl_bwd_shard(H, W, 0, I, A, M, tau, None, lse, g, dH, dW, chunk_rows, ws)

    kd.kd_topk_kl_fwd_shard(H, W, 0, I, A, M, tau, None, rec[0], trow, None, ws)
    rec[1:].copy_(rec[0].expand(R - 1, T, 4))
    step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base + (rec.numel() + trow.numel() + lse.numel()) * 4
    ms, prof, ksteps = timed(step, steps, warmup)
    fl = {k: 2.0 * n_valid * d * Vs for k in ("topk_fwd_tile", "topk_dz_tile", "dh_tile", "dw_tile")}
    dom, achieved = dominant(prof, fl, ksteps)
    cred = 6.0 * n_valid * d * Vs / (ms * 1e-3) / 1e12
    out = {"workload": f"{p.name}_vshard{R}", "T": T, "V_shard": Vs, "valid_rows": n_valid, "ms_per_step": ms,
           "tokens_per_s": T / (ms * 1e-3), "valid_tokens_per_s": n_valid / (ms * 1e-3), "credited_tflops": cred,
           "mfma_frac_credited": cred / PEAK_BF16_TFLOPS, "mfma_frac_executed": cred / PEAK_BF16_TFLOPS * 8.0 / 6.0,
           "peak_extra_hbm_bytes": int(peak_extra), "dominant": dom, "dominant_tflops": achieved,
           "kernels": kernel_table(prof, ksteps), "steps_timed": steps}
    del H, W, I, A, g, M, rec, trow, kl, lse, dH, dW, ws
    torch.cuda.empty_cache()
    return out


def run_full_shard(p, R: int, steps: int, warmup: int, chunk_rows: int):
    """Time one rank's step of the full-vocabulary loss with both heads split
    by vocabulary over R ranks (rank 0: columns [0, V/R) of each head): its
    forward, the combine of R records and its backward.  As in
    run_topk_shard, the other ranks' records are copies of its own, made once
    before timing."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    T, d, dt, tau = p.T, p.d, p.dt_hidden, p.tau
    Vs = p.V // R
    inp = G.make_full(T, d, dt, p.V, p.dtype, tau=tau, number=p.number, g="mean")
    dev = torch.device("cuda:0")
    H, Ht, g = (inp[k].to(dev) for k in ("H", "Ht", "g"))
    Ws = inp["Ws"][:, :Vs].contiguous().to(dev)
    Wt = inp["Wt"][:, :Vs].contiguous().to(dev)
    del inp
    rec = torch.empty(R, T, 8, device=dev)
    kl, ls, lt = (torch.empty(T, device=dev) for _ in range(3))
    dH = torch.empty(T, d, device=dev)
    dW = torch.empty(d, Vs, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    ws = torch.empty(kd.kd_full_kl_workspace_size(T, d, dt, Vs, p.dtype, chunk_rows), dtype=torch.uint8, device=dev)

    def step():
        kd.kd_full_kl_fwd_shard(H, Ws, Ht, Wt, None, tau, None, rec[0], ws)
        kd.kd_full_kl_shard_combine(rec, None, 0.0, kl, ls, lt, None)
        kd.kd_full_kl_bwd_shard(H, Ws, Ht, Wt, None, tau, None, ls, lt, None, g, dH, dW, chunk_rows, ws)

    kd.kd_full_kl_fwd_shard(H, Ws, Ht, Wt, None, tau, None, rec[0], ws)
    rec[1:].copy_(rec[0].expand(R - 1, T, 8))
    step()
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base + (rec.numel() + 2 * T) * 4
    ms, prof, ksteps = timed(step, steps, warmup)
    fl = {"full_fwd_tile": 2.0 * T * (d + dt) * Vs, "full_dz_tile": 2.0 * T * (d + dt) * Vs,
          "dh_tile": 2.0 * T * d * Vs, "dw_tile": 2.0 * T * d * Vs}
    dom, achieved = dominant(prof, fl, ksteps)
    cred = (2.0 * (d + dt) * Vs + 4.0 * d * Vs) * T / (ms * 1e-3) / 1e12
    out = {"workload": f"{p.name}_vshard{R}", "T": T, "V_shard": Vs, "ms_per_step": ms,
           "tokens_per_s": T / (ms * 1e-3), "credited_tflops": cred, "mfma_frac_credited": cred / PEAK_BF16_TFLOPS,
           "peak_extra_hbm_bytes": int(peak_extra), "dominant": dom, "dominant_tflops": achieved,
           "kernels": kernel_table(prof, ksteps), "steps_timed": steps}
    del H, Ht, g, Ws, Wt, rec, kl, ls, lt, dH, dW, ws
    torch.cuda.empty_cache()
    return out


def progress(msg: str):
    """One line on stderr per finished workload (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def brief(r):
    progress(f"{r['workload']}: {r['ms_per_step']:.3f} ms per step")
    keep = ("workload", "T", "V_shard", "valid_rows", "ms_per_step", "tokens_per_s", "valid_tokens_per_s", "credited_tflops",
            "mfma_frac_credited", "mfma_frac_executed", "peak_extra_hbm_bytes", "dominant", "dominant_tflops")
    out = {k: r[k] for k in keep if k in r}
    out["kernel_ms"] = {k: round(v["ms_per_step"], 4) for k, v in r["kernels"].items()} if "kernels" in r else None
    return out


def vendor_gemm(steps: int, warmup: int):
    """The vendor BLAS GEMM (torch.matmul, bf16 in) on the three contractions of
    the head's step: H.W (forward and the backward's recompute), dZ.W^T (dH)
    and H^T.dZ (dW, bf16 out, then also into an fp32 array as the loss's dW
    is).  Plain products with no loss epilogue: a reference for what this chip
    sustains on these shapes at its loaded clock, timed like the loss steps."""
    import torch
    dev = torch.device("cuda:0")
    T, d, V = 4096, 3072, 128256
    gen = torch.Generator(device=dev).manual_seed(7)
    H = torch.randn(T, d, device=dev, dtype=torch.bfloat16, generator=gen)
    W = (torch.randn(d, V, device=dev, dtype=torch.bfloat16, generator=gen) / d ** 0.5).to(torch.bfloat16)
    dZ = (torch.randn(T, V, device=dev, dtype=torch.bfloat16, generator=gen) * 1e-3).to(torch.bfloat16)
    Z = torch.empty(T, V, device=dev, dtype=torch.bfloat16)
    dWf = torch.empty(d, V, device=dev, dtype=torch.float32)
    flops = 2 * T * d * V
    cases = (("H.W -> bf16 [T,V]", lambda: torch.matmul(H, W, out=Z)),
             ("dZ.W^T -> bf16 [T,d]", lambda: torch.matmul(dZ, W.t())),  # plain 2-D product, W read in place
             ("H^T.dZ -> bf16 [d,V]", lambda: torch.matmul(H.t(), dZ)),
             ("H^T.dZ -> fp32 [d,V] (bf16 product, then copied)", lambda: dWf.copy_(torch.matmul(H.t(), dZ))))
    for name, f in cases:
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            f()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        print(json.dumps({"vendor_gemm": name, "T": T, "d": d, "V": V, "ms": round(ms, 4),
                          "tflops": round(flops / ms / 1e9, 1), "frac_of_2.5PF": round(flops / ms / 1e9 / 2500, 4)}),
              flush=True)


def operand_probe(kind: str, steps: int, warmup: int):
    """The headline workload's forward and backward calls on its seeded
    operands, or with H and W all zero.  The kernels run the same
    instructions either way; under matrix load the chip's clock follows the
    power its operands draw, so the two show how much of the distance to the
    published peak is the clock rather than the kernels' share of busy
    cycles (read with rocprofv3 counters).  Prints one diagnostic line."""
    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G
    p = G.PRESETS["head_topk_t4096"]
    inp = G.make_preset(p, g="mean")
    dev = torch.device("cuda:0")
    H, W, I, A, g = (inp[k].to(dev) for k in ("H", "W", "I", "A", "g"))
    del inp
    if kind == "zero":
        H.zero_()
        W.zero_()
    T, d, V, K = p.T, p.d, p.V, p.K
    kl, lse = torch.empty(T, device=dev), torch.empty(T, device=dev)
    dH, dW = torch.empty_like(H), torch.empty(d, V, device=dev)
    ws = torch.empty(kd.kd_topk_kl_workspace_size(T, d, V, K, p.dtype, 0), dtype=torch.uint8, device=dev)

    def step():
        kd.kd_topk_kl_fwd(H, W, I, A, None, p.tau, kl, lse, None, ws)
        kd.kd_topk_kl_bwd(H, W, I, A, None, p.tau, lse, g, dH, dW, 0, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    print(json.dumps({"operand_probe": kind, "workload": p.name, "steps": steps, "ms_per_step": round(ms, 4),
                      "note": "diagnostic of the clock's dependence on the operands; not the metric"}), flush=True)


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.vendor_gemm:
        vendor_gemm(a.steps, a.warmup)
        return
    if a.operand_probe:
        operand_probe(a.operand_probe, a.steps, a.warmup)
        return

    import kdinputs as G

    if a.sweep:
        for T in G.SWEEP_T:
            p = G.sweep_preset(T)
            steps = max(2, min(a.steps, (4 * 4096 * 10) // T))
            r, _ = run_topk(p, T, steps, 1, a.chunk_rows)
            print(json.dumps({"sweep": p.name, "steps": steps, **brief(r)}), flush=True)
        return

    if a.workload.endswith("_vshard8"):  # one rank's step of an 8-way vocabulary split, on its own
        base = G.PRESETS.get(a.workload[:-len("_vshard8")])
        if base is None:
            print(f"unknown workload {a.workload}", file=sys.stderr)
            sys.exit(2)
        r = (run_full_shard(base, 8, a.steps, a.warmup, a.chunk_rows) if base.full_vocab
             else run_topk_shard(base, base.T, 8, a.steps, a.warmup, a.chunk_rows))
        print(json.dumps({"metric": "one rank's fwd+bwd tokens/s, head split 8 ways by vocabulary",
                          "value": r["tokens_per_s"], "unit": "tokens/s", **brief(r)}))
        return

    p = G.PRESETS.get(a.workload)
    if p is None:
        print(f"unknown workload {a.workload}", file=sys.stderr)
        sys.exit(2)
    if p.full_vocab:
        r = run_full(p, a.steps, a.warmup, a.chunk_rows, a.one_call)
        print(json.dumps({"metric": "full-vocab KL fwd+bwd tokens/s", "value": r["tokens_per_s"],
                          "unit": "tokens/s", **brief(r)}))
        return

    T = a.T or p.T
    r, inp = run_topk(p, T, a.steps, a.warmup, a.chunk_rows, protocol=not a.no_protocol)
    progress(f"{p.name}: {r['ms_per_step']:.3f} ms per step")
    workload = p.name if not a.T else f"{p.name}_T{T}"
    dom = r["dominant"]
    n_l = r["kernels"][dom]["launches"]
    rows_per_launch = r["valid_rows"] if dom == "topk_fwd_tile" else r["valid_rows"] / (n_l / a.steps)
    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "T": T, "d": p.d, "V": p.V, "K": p.K, "tau": p.tau,
                   "valid_rows": r["valid_rows"], "chunk_rows": a.chunk_rows or 4096},
        "valid_tokens_per_s": r["valid_tokens_per_s"],
        "credited_tflops": r["credited_tflops"],
        "mfma_frac_credited": r["mfma_frac_credited"],
        "mfma_frac_executed": r["mfma_frac_executed"],
        "peak_extra_hbm_bytes": r["peak_extra_hbm_bytes"],
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": r["dominant_tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": r["dominant_tflops"] / PEAK_BF16_TFLOPS,
                     "source": "the tile kernel with the most time in a pass of its own after the timed steps, "
                               "each launch timed by HIP events on its stream",
                     "traffic": traffic_from_profiles(dom, workload),
                     "flops_per_launch": 2.0 * rows_per_launch * p.d * p.V},
        "kernels": r["kernels"],
    }
    if "pages_protocol" in r:
        out["pages_protocol"] = r["pages_protocol"]
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, min(a.cpu_rows, T))
        progress(f"oracle on the host: {out['cpu_baseline']['sample']}")
    del inp
    if not a.no_extra and not a.T and a.workload == "head_topk_t4096":
        pk = G.PRESETS["head_topk_t32768_packed"]
        fv = G.PRESETS["full_vocab_t16384"]
        one = run_topk_fused(p, T, a.steps, a.warmup, a.chunk_rows)
        out["extra"] = {one["workload"]: brief(one),
                        pk.name: brief(run_topk(pk, pk.T, 3, 1, a.chunk_rows)[0]),
                        fv.name: brief(run_full(fv, 3, 1, a.chunk_rows)),
                        fv.name + "_one_call": brief(run_full(fv, 3, 1, a.chunk_rows, one_call=True))}
        pk16 = brief(run_topk(pk, pk.T, 3, 1, 16384)[0])
        pk16["workload"] = pk.name + "_chunk16384"
        out["extra"][pk16["workload"]] = pk16
        sh = run_topk_shard(p, T, 8, a.steps, a.warmup, a.chunk_rows)
        out["extra"][sh["workload"]] = brief(sh)
        fs = run_full_shard(fv, 8, 3, 1, a.chunk_rows)
        out["extra"][fs["workload"]] = brief(fs)
        # the loss-only sweep's longer points: throughput and peak extra HBM,
        # which must grow linearly in T (no [T, V] buffer anywhere)
        pts = [(T, r["peak_extra_hbm_bytes"])]
        for Ts in G.SWEEP_T:
            if Ts == T:
                continue
            sw = brief(run_topk(G.sweep_preset(Ts), Ts, 2, 1, a.chunk_rows)[0])
            out["extra"][sw["workload"]] = sw
            pts.append((Ts, sw["peak_extra_hbm_bytes"]))
        out["extra"]["peak_extra_hbm_fit"] = linear_fit(pts)
    print(json.dumps(out))


def linear_fit(pts):
    """Least-squares a + b T through (T, bytes) points, and the largest
    relative residual."""
    n = len(pts)
    mt = sum(t for t, _ in pts) / n
    mb = sum(b for _, b in pts) / n
    b = sum((t - mt) * (y - mb) for t, y in pts) / sum((t - mt) ** 2 for t, _ in pts)
    a0 = mb - b * mt
    res = max(abs(a0 + b * t - y) / y for t, y in pts)
    return {"points": [[t, y] for t, y in sorted(pts)], "bytes_const": a0, "bytes_per_token": b,
            "max_rel_residual": res}


if __name__ == "__main__":
    main()
