"""Throughput of the fused top-K KL loss, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one kd_topk_kl_fwd plus one kd_topk_kl_bwd over one batch of
synthetic rows (inputs already in HBM): the output projection, online log Z,
top-K gather, per-token KL, and the chunked backward (recomputed projection,
dZ, dH, dW).  Prints one JSON line.

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
PEAK_HBM_GBS = 8000.0
TILE_KERNELS = ("topk_fwd_tile", "topk_dz_tile", "dh_tile", "dw_tile")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="head_topk_t4096")
    ap.add_argument("--T", type=int, default=0, help="override the row count (sweep)")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 4 times (calibrates HBM byte counters)")
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
    import numpy as np
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
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} of {inp['H'].shape[0]} rows, forward + backward, fp64 NumPy "
                      f"(BLAS threads = cores), {dt:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if a.copy_probe:
        copy_probe(a.copy_probe)
        return

    import torch
    import chunked_kl_loss_logit_amd as kd
    import kdinputs as G

    p = G.PRESETS[a.workload] if a.workload in G.PRESETS else None
    if p is None or p.full_vocab:
        print(f"unknown top-K workload {a.workload}", file=sys.stderr)
        sys.exit(2)
    T = a.T or p.T
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
    ws = torch.empty(kd.kd_topk_kl_workspace_size(T, d, V, K, p.dtype, a.chunk_rows), dtype=torch.uint8, device=dev)
    kd.kd_topk_kl_fwd(H, W, I, A, M, tau, kl, lse, None, ws)
    kd.kd_topk_kl_bwd(H, W, I, A, M, tau, lse, g, dH, dW, a.chunk_rows, ws)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - base + lse.numel() * 4  # + saved lse

    def step():
        kd.kd_topk_kl_fwd(H, W, I, A, M, tau, kl, lse, None, ws)
        kd.kd_topk_kl_bwd(H, W, I, A, M, tau, lse, g, dH, dW, a.chunk_rows, ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    kd.profile_reset()
    kd.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kd.profile_enable(False)
    prof = kd.profile_read()
    print(f"[bench] {a.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    ms = elapsed / a.steps * 1e3
    credited = 6.0 * n_valid * d * V          # 2dV forward + 4dV backward per token
    executed = 8.0 * n_valid * d * V          # the backward recomputes the projection
    tflops = credited / (ms * 1e-3) / 1e12
    per_kernel = {k: {"launches": n, "avg_ms": tot / n, "share": tot / (ms * a.steps)} for k, (n, tot) in prof.items()}
    dom = max((k for k in prof if k in TILE_KERNELS), key=lambda k: prof[k][1])
    n_l, tot_ms = prof[dom]
    avg_ms = tot_ms / n_l
    # each tile kernel contracts one chunk: 2 * rows * d * V flops per launch
    rows_per_launch = n_valid if dom == "topk_fwd_tile" else n_valid / (n_l / a.steps)
    achieved = 2.0 * rows_per_launch * d * V / (avg_ms * 1e-3) / 1e12
    workload = p.name if not a.T else f"head_topk_t{T}"
    traffic = traffic_from_profiles(dom, workload)

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "T": T, "d": d, "V": V, "K": K,
                   "tau": tau, "valid_rows": n_valid, "chunk_rows": a.chunk_rows or 4096},
        "valid_tokens_per_s": n_valid / (ms * 1e-3),
        "credited_tflops": tflops,
        "mfma_frac_credited": tflops / PEAK_BF16_TFLOPS,
        "mfma_frac_executed": executed / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "peak_extra_hbm_bytes": int(peak_extra),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic},
        "kernels": per_kernel,
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, min(a.cpu_rows, T))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
