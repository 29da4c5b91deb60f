#!/usr/bin/env python3
"""Benchmark one SparsePR attention call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3_dit_32k]

A step is one full call (partitioning, routing, permutation, probes, fit,
sparse attention with the fused correction, output restoration) over one
synthetic [1, H, N, d] bf16 input resident in HBM.  Prints ONE JSON line with
ms/call, executed-pair TFLOP/s, the dense-attention time at the same shape
(the faster of torch SDPA and the library's own dense kernel), the roofline
of the dominant kernel (block-sparse attention, timed with HIP events on the
library's stream) and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector: 256 CUs x 128 FMA per clock x 2 flops x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3_dit_32k")
    ap.add_argument("--density", type=float, default=None)
    ap.add_argument("--router", choices=("budget", "alpha"), default="budget",
                    help="cell selection: pair budget from the density, or per-group target retained mass")
    ap.add_argument("--alpha", type=float, default=0.9, help="target retained mass of --router alpha")
    ap.add_argument("--diagnostics", action="store_true",
                    help="structural diagnostics of both partitions (support, affine-explainable residual)")
    ap.add_argument("--diag-heads", type=int, default=4, help="heads measured by --diagnostics")
    ap.add_argument("--diag-rows", type=int, default=8, help="measured queries per query group")
    ap.add_argument("--rank-cap", type=float, default=1.0, help="residual rank at most floor(cap * M)")
    ap.add_argument("--svd-weighted", action="store_true", help="residual subspace from the weighted SVD")
    ap.add_argument("--centred", action="store_true", help="centred query coordinates")
    ap.add_argument("--sweep", choices=("density", "probes", "headdim", "all"), default=None,
                    help="instead of the bench line: one JSON line per point of a quality/efficiency sweep "
                         "(both partitions; ms/call, rho_exec, corrected and hard-drop error vs dense)")
    ap.add_argument("--densities", default="0.10,0.12,0.15,0.18,0.21,0.22,0.25,0.26,0.30,0.35,0.40")
    ap.add_argument("--probe-budgets", default="16,32,64,128,256")
    ap.add_argument("--gen-device", choices=("cpu", "cuda"), default="cpu",
                    help="where the seeded generator runs its per-head projections (cuda: seconds instead of "
                         "minutes at 75k tokens; the host draws are the same)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--profile-runs", type=int, default=3, help="calls timed per stage (at least 1)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration) and exit")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_sparse_attention.json"))
    return ap.parse_args()


def time_fn(fn, reps: int, torch) -> list:
    """Per-call milliseconds of fn() on the current stream (HIP events)."""
    out = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        out.append(a.elapsed_time(b))
    return out


def cpu_baseline(x, w, cfg_kw, n: int, d: int, m: int, heads: int = 4) -> dict:
    """Time the oracle on the first `heads` heads (a bounded sample of the call)."""
    try:
        from threadpoolctl import threadpool_info
    except Exception:  # pragma: no cover
        threadpool_info = None
    from oracle import OracleConfig, sparsepr_head

    cfg = OracleConfig(**cfg_kw)
    heads = min(heads, w.heads)
    pairs = 0
    t0 = time.perf_counter()
    for h in range(heads):
        q = x["q"][0, h].double().cpu().numpy()
        k = x["k"][0, h].double().cpu().numpy()
        v = x["v"][0, h].double().cpu().numpy()
        r = sparsepr_head(q, k, v, cfg, bh=h)
        pairs += r["route"]["routed_pairs"] + m * n
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    if threadpool_info is not None:
        th = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if th:
            cores = max(th)
    return {"value": 4.0 * d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"heads 0-{heads - 1} of {w.heads} of {w.name} (full per-head calls, {dt:.1f} s)",
            "seconds": round(dt, 3)}


def sweep(args, sp, torch, w, x) -> int:
    """Quality/efficiency sweep of both partitions against the library's dense output."""
    from synth import make_workload_inputs

    points = []  # (axis, d, density, probe rows)
    if args.sweep in ("density", "all"):
        points += [("density", w.d, float(r), w.probe_rows) for r in args.densities.split(",")]
    if args.sweep in ("probes", "all"):
        points += [("probes", w.d, w.density, int(m)) for m in args.probe_budgets.split(",")]
    if args.sweep in ("headdim", "all"):
        points += [("headdim", dd, w.density, w.probe_rows) for dd in (64, 128)]
    ws = sp.Workspace()
    cache = {}
    for axis, dd, rho, m in points:
        if dd not in cache:
            xx = x if dd == w.d else make_workload_inputs(w, d=dd, device=args.gen_device)
            q, k, v = (xx[t].cuda() for t in ("q", "k", "v"))
            dense = sp.sparsepr_dense_attention(q, k, v).float()
            cache.clear()
            cache[dd] = (q, k, v, dense, float(dense.norm()))
        q, k, v, dense, dn = cache[dd]
        B, H, N, _ = q.shape
        out = torch.empty_like(q)
        for mode in ("response_coupled", "independent"):
            cfg = sp.make_config(N, dd, density=rho, probe_rows=m, n_kv_groups=w.n_kv_groups,
                                 n_q_groups=w.n_q_groups, residual_rank=w.residual_rank, partition_mode=mode,
                                 rank_cap=args.rank_cap, svd_weighted=int(args.svd_weighted),
                                 centred_query_coords=int(args.centred))
            sp.sparsepr_attention(q, k, v, cfg, out=out, workspace=ws)  # warm-up
            ms = min(time_fn(lambda: sp.sparsepr_attention(q, k, v, cfg, out=out, workspace=ws), 3, torch))
            _, _, st = sp.sparsepr_attention_profile(q, k, v, cfg, out=out, workspace=ws)
            heads = sp.stats_to_dicts(st)
            err = float((out.float() - dense).norm()) / dn
            ql, kl = sp.sparsepr_partition(q, k, v, cfg, workspace=ws)
            hard = sp.sparsepr_sparse_attention(q, k, v, cfg, ql, kl, workspace=ws)
            herr = float((hard.float() - dense).norm()) / dn
            rho_exec = sum(h["routed_pairs"] + h["probe_pairs"] for h in heads) / (B * H * N * N)
            print(json.dumps({"sweep": axis, "workload": w.name, "partition": mode, "d": dd, "density": rho,
                              "probe_rows": m, "rank_cap": args.rank_cap, "svd_weighted": bool(args.svd_weighted),
                              "centred": bool(args.centred), "rho_exec": round(rho_exec, 5),
                              "ms_per_call": round(ms, 4),
                              "rel_err_corrected": round(err, 5), "rel_err_hard_drop": round(herr, 5)}), flush=True)
            log(f"{axis} {mode} d {dd} rho {rho} M {m}: {ms:.2f} ms, err {err:.4f} (hard drop {herr:.4f})")
    return 0


def diagnostics(args, sp, torch, w, x) -> int:
    """Structural diagnostics of both partitions on the first heads of the workload."""
    import numpy as np
    from free_block_sparse_amd.diagnostics import structural_diagnostics

    hh = min(args.diag_heads, w.heads)
    q, k, v = (x[t][:, :hh].contiguous().cuda() for t in ("q", "k", "v"))
    B, H, N, d = q.shape
    rng = np.random.default_rng(0)
    for mode in ("response_coupled", "independent"):
        cfg = sp.make_config(N, d, density=w.density, probe_rows=w.probe_rows, n_kv_groups=w.n_kv_groups,
                             n_q_groups=w.n_q_groups, residual_rank=w.residual_rank, partition_mode=mode)
        ql, _ = sp.sparsepr_partition(q, k, v, cfg)
        # the same number of measured queries from every query group of head 0
        lab = ql[0].cpu().numpy()
        rows = []
        for g in np.unique(lab):
            members = np.nonzero(lab == g)[0]
            rows += list(rng.choice(members, size=min(args.diag_rows, members.size), replace=False))
        t0 = time.time()
        res = structural_diagnostics(q, k, v, cfg, rows=sorted(int(r) for r in rows))
        for h, r in enumerate(res):
            print(json.dumps({"diagnostics": mode, "workload": w.name, "head": h, "density": w.density,
                              "measured_rows": len(rows), **{kk: round(vv, 5) for kk, vv in r.items()}}),
                  flush=True)
        log(f"diagnostics {mode}: {len(res)} heads in {time.time() - t0:.1f}s")
    return 0


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; multi-GPU runs are not supported (use --gpus 1)"}))
        log("only --gpus 1 is supported: the call runs on one GPU (heads would shard across GPUs without exchange)")
        return 2
    n_threads = len(os.sched_getaffinity(0))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, str(n_threads))

    import torch
    import free_block_sparse_amd as sp
    from synth import make_workload_inputs, workload

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 3}), flush=True)
        return 0
    w = workload(args.workload)
    if args.density is not None:
        w = workload(args.workload, density=args.density)
    log(f"generating inputs for {w.name}: H={w.heads} N={w.n} d={w.d} {w.dtype}")
    t0 = time.time()
    x = make_workload_inputs(w, device=args.gen_device)
    log(f"inputs ready in {time.time() - t0:.1f}s")
    if args.sweep:
        return sweep(args, sp, torch, w, x)
    if args.diagnostics:
        return diagnostics(args, sp, torch, w, x)
    q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
    B, H, N, d = q.shape
    cfg_kw = dict(density=w.density, probe_rows=w.probe_rows, n_kv_groups=w.n_kv_groups,
                  n_q_groups=w.n_q_groups, residual_rank=w.residual_rank, router=args.router, alpha=args.alpha)
    cfg = sp.make_config(N, d, **cfg_kw)
    ws = sp.Workspace()
    out = torch.empty_like(q)

    def call():
        sp.sparsepr_attention(q, k, v, cfg, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} calls)")
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    ms_call = start.elapsed_time(stop) / args.steps
    log(f"timed {args.steps} calls: {ms_call:.3f} ms/call")

    # per-stage times (HIP events on the library's stream) and statistics
    stage_runs = []
    stats = None
    for _ in range(max(1, args.profile_runs)):
        _, st_ms, st = sp.sparsepr_attention_profile(q, k, v, cfg, out=out, workspace=ws)
        stage_runs.append(st_ms)
        stats = st
    torch.cuda.synchronize()
    stage_ms = {s: sum(r[s] for r in stage_runs) / len(stage_runs) for s in stage_runs[0]}
    heads = sp.stats_to_dicts(stats)
    routed = sum(h["routed_pairs"] for h in heads)
    probe_pairs = sum(h["probe_pairs"] for h in heads)
    rho_exec = (routed + probe_pairs) / (B * H * N * N)
    kernel_flops = 4.0 * d * routed
    call_flops = 4.0 * d * (routed + probe_pairs)
    t_kernel = stage_ms["sparse_attention"]
    kernel_tflops = kernel_flops / (t_kernel * 1e-3) / 1e12
    call_tflops = call_flops / (ms_call * 1e-3) / 1e12
    log(f"stages (ms): " + ", ".join(f"{s}={v:.3f}" for s, v in stage_ms.items()))

    result_extra = {}
    if not args.no_dense:
        import torch.nn.functional as F
        dense_out = torch.empty_like(q)
        sdpa_ms = time_fn(lambda: F.scaled_dot_product_attention(q, k, v), 3, torch)
        own_ms = time_fn(lambda: sp.sparsepr_dense_attention(q, k, v, out=dense_out), 3, torch)
        ref = F.scaled_dot_product_attention(q, k, v).float()
        err = float((out.float() - ref).norm() / ref.norm())
        # the uncorrected (hard-drop) output of the same partition, for comparison
        ql, kl = sp.sparsepr_partition(q, k, v, cfg, workspace=ws)
        hard = sp.sparsepr_sparse_attention(q, k, v, cfg, ql, kl, workspace=ws)
        herr = float((hard.float() - ref).norm() / ref.norm())
        del hard, ql, kl
        dense_ms = min(min(sdpa_ms), min(own_ms))
        result_extra.update(dense_ms=round(dense_ms, 4), dense_ms_torch_sdpa=round(min(sdpa_ms), 4),
                            dense_ms_own_kernel=round(min(own_ms), 4),
                            speedup_vs_dense=round(dense_ms / ms_call, 4), rel_err_vs_dense=round(err, 5),
                            rel_err_hard_drop=round(herr, 5))
        log(f"dense: sdpa {min(sdpa_ms):.3f} ms, own {min(own_ms):.3f} ms; speedup {dense_ms / ms_call:.3f}; "
            f"rel err vs dense {err:.4f} (hard drop {herr:.4f})")
        del dense_out, ref

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("workload") == w.name and tj.get("kernel_source_sha") == _kernel_sha():
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the first heads (bounded sample)")
        cpu = cpu_baseline(x, w, cfg_kw, N, d, w.probe_rows)
        log(f"oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads ({cpu['seconds']} s)")

    res = {
        "metric": "ms/call & executed-pair TFLOP/s (%bf16 MFMA peak) at 25% density; speedup vs dense",
        "value": round(call_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "fp32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "density": w.density,
                   "n_kv_groups": w.n_kv_groups, "n_q_groups": w.n_q_groups, "probe_rows": w.probe_rows,
                   "residual_rank": w.residual_rank, "kmeans_iters": cfg.kmeans_iters, "router": args.router,
                   **({"alpha": args.alpha} if args.router == "alpha" else {}), "parallelism": "none"},
        "roofline": ({"bound": "mfma", "achieved": round(kernel_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                      "kernel": "k_sparse_attn_mfma (block-sparse attention, fused correction)",
                      "kernel_ms": round(t_kernel, 4), "flops_per_launch": kernel_flops}
                     if w.dtype != "fp32" else
                     {"bound": "alu", "achieved": round(kernel_tflops, 2), "peak": PEAK_FP32_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(kernel_tflops / PEAK_FP32_TFLOPS, 4), "traffic": None,
                      "kernel": "k_sparse_attn_vec (fp32 block-sparse attention, fused correction)",
                      "kernel_ms": round(t_kernel, 4), "flops_per_launch": kernel_flops}),
        "cpu_baseline": cpu,
        "call_pct_peak": round(100 * call_tflops / PEAK_BF16_TFLOPS, 2),
        "rho_exec": round(rho_exec, 5),
        "rho_route": round(routed / (B * H * N * N), 5),
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
    }
    res.update(result_extra)
    print(json.dumps(res), flush=True)
    return 0


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha1()
    p = os.path.join(ROOT, "free_block_sparse_amd", "csrc", "k_attn.hip")
    h.update(open(p, "rb").read())
    return h.hexdigest()[:12]


if __name__ == "__main__":
    sys.exit(main())
