"""Benchmark of the fused ranking head (scores + logsumexp + top-K) on one GPU.

Default workload: 1,024 users x 1,000,000 items, D = 4,096, K = 500, bf16
(the large compute-bound catalog).  One step = one full call of the head on
inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload large|batch|gemv|tiny|cand]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("user×item scores/sec (TFLOP/s) for fused score+lse+top-K; "
          "% of MFMA/HBM roofline")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_MATRIX_PEAK_TFLOPS = 157.3  # dense fp32 on the matrix cores


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_steps(torch, step, steps):
    """Times `steps` calls of step() back to back: the mean over the whole
    bracketed region (synchronised before and after), and the median and
    minimum of the per-step intervals between events recorded on the stream
    in between (no synchronisation inside the region)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mean = ev[0].elapsed_time(ev[steps]) / steps
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return mean, med, per[0]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large",
                    choices=["large", "batch", "batch_f32", "gemv", "tiny", "cand", "gemv_big", "beam128", "beam512",
                             "ce"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target host time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--de-dtype", default="f32", choices=["f32", "bf16"],
                    help="ce workload: dtype of the catalog gradient dE")
    ap.add_argument("--mask-density", type=float, default=None, metavar="P",
                    help="full-catalog workloads: score through the masked head with one seeded "
                         "item mask that allows a fraction P of the catalog")
    ap.add_argument("--clusters", type=int, default=0, metavar="C",
                    help="full-catalog workloads: a catalog stored grouped by category (C clusters of "
                         "contiguous ids, synth.gen_E_clustered) instead of the exchangeable one; the line "
                         "reports how many users the call rescued")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scratch buffer before every step (flushes the 256 MB Infinity "
                         "Cache and the L2s) and time each step on its own, the flush outside")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured as a HIP graph (the same launches without the "
                         "host call's cost); per-kernel times still come from eager steps")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure library reference rates on this GPU (device copy GB/s, "
                         "hipBLASLt bf16 GEMM TFLOP/s) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (the reference "
                         "kernel for scaling HBM byte counters) and exit")
    return ap.parse_args()


def to_dev(a, dev, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def copy_calibration(mib, reps):
    """Plain copies of a known size: FETCH_SIZE / WRITE_SIZE of this kernel against its
    exact byte count give the scale of those counters."""
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def peaks(emit=True):
    """Reference rates of this GPU from library code: a 4 GiB device-to-device copy
    (bytes read + written / time) and torch.matmul (hipBLASLt) of bf16 8192^3 with
    the second operand transposed (both operands K-contiguous, like H and E)."""
    import torch
    dev = torch.device("cuda:0")
    out = {}
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["device_copy_GBps"] = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    bt = b.t()
    for _ in range(3):
        c = a @ bt
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        c = a @ bt
    e1.record()
    torch.cuda.synchronize()
    out["hipblaslt_bf16_8192_NT_TFLOPs"] = 2 * 8192 ** 3 * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del c, a, b, bt
    torch.cuda.empty_cache()
    out["kind"] = "library reference rates on this GPU (not the spec peaks)"
    if emit:
        print(json.dumps({"peaks": out}), flush=True)
    return out


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary,
    or None when the summary is absent or was taken from other kernel sources."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.md" % (kernel, workload))
    src = os.path.join(ROOT, "full_catalog_ranking_amd", "csrc", "kernels.hip")
    if not os.path.exists(path):
        return None
    want = hashlib.sha256(open(src, "rb").read()).hexdigest()
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernels.hip sha256") != want:
        return None
    try:
        return float(fields["hbm bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(d, K, target_s, cand, mask_words=None):
    """The oracle on a bounded sample of the same workload: whole users."""
    from oracle import oracle
    oracle.build()
    B = d["B"]
    users = [0]

    def dense(us):
        if mask_words is None:
            oracle.full(d["H"], d["E"], K, users=us)
        else:
            oracle.full_masked(d["H"], d["E"], K, mask_words, users=us)

    t0 = time.perf_counter()
    if cand:
        oracle.cand(d["H"], d["E"], d["offsets"], d["ids"], K, users=users)
    else:
        dense(users)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(B, target_s / max(t1, 1e-3))))
    users = list(np.linspace(0, B - 1, n).astype(np.int64))
    t0 = time.perf_counter()
    if cand:
        oracle.cand(d["H"], d["E"], d["offsets"], d["ids"], K, users=users)
        units = int(sum(d["offsets"][u + 1] - d["offsets"][u] for u in users))
    else:
        dense(users)
        units = n * d["M"]
    t = time.perf_counter() - t0
    return dict(value=units / t, unit="scores/s", cores=oracle.threads(), kind="oracle",
                sample="%d of %d users, %d scores with lse and full sort, %.1f s" % (n, B, units, t))


def bench_beam(args):
    """Beam step: batched top-K of R dense score rows of N entries (one call)."""
    import torch
    from full_catalog_ranking_amd import genrec, synth
    dev = torch.device("cuda:0")
    genrec.lib()
    d = synth.make_workload(args.workload)
    R, N, K = d["R"], d["N"], d["K"]
    S = torch.from_numpy(d["scores"]).to(dev)
    out = (torch.empty((R, K), dtype=torch.int32, device=dev), torch.empty((R, K), dtype=torch.float32, device=dev))
    for _ in range(args.warmup):
        genrec.topk_rows(S, K, out=out)
    torch.cuda.synchronize()
    ms, med, mn = timed_steps(torch, lambda: genrec.topk_rows(S, K, out=out), args.steps)
    alg_bytes = R * N * 4 + R * K * 8
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": R * N / (ms * 1e-3), "unit": "scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": med,
        "ms_per_step_min": mn, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "R": R, "N": N, "K": K},
        # the whole call, every pass of its route (per chunk or segment, then
        # per row; or sample, filter and list ranking), timed with events on
        # the stream they run on
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "kernel": "genrec_topk_rows (every pass)", "kernel_ms": ms,
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle
        oracle.build()
        t0 = time.perf_counter()
        oracle.topk_row(d["scores"][0].astype(np.float64), K)
        t1 = max(time.perf_counter() - t0, 1e-4)
        n = int(max(1, min(R, args.cpu_seconds / t1)))
        t0 = time.perf_counter()
        for r in np.linspace(0, R - 1, n).astype(np.int64):
            oracle.topk_row(d["scores"][r].astype(np.float64), K)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=n * N / t, unit="scores/s", cores=1, kind="oracle",
                                   sample="%d of %d rows, full stable sort each, %.1f s" % (n, R, t))
    print(json.dumps(res), flush=True)


def bench_ce(args):
    """Reward-weighted catalog cross-entropy: one step = forward + backward."""
    import torch
    from full_catalog_ranking_amd import genrec, synth
    dev = torch.device("cuda:0")
    genrec.lib()
    t0 = time.perf_counter()
    if args.clusters and (args.workload in ("cand", "tiny") or cfg.get("kind")):
        raise SystemExit("--clusters applies to the full-catalog workloads")
    d = synth.make_workload(args.workload, **({"clusters": args.clusters} if args.clusters else {}))
    log("inputs generated in %.1f s" % (time.perf_counter() - t0))
    B, D, M = d["B"], d["D"], d["M"]
    H, E = to_dev(d["H"], dev, torch), to_dev(d["E"], dev, torch)
    lab = torch.from_numpy(d["labels"]).to(dev)
    w = torch.from_numpy(d["weights"]).to(dev)
    wsf = torch.empty(genrec.lib().genrec_ce_forward_workspace(B, D, M), dtype=torch.uint8, device=dev)
    wsb = torch.empty(genrec.lib().genrec_ce_backward_workspace(B, D, M), dtype=torch.uint8, device=dev)
    dH = torch.empty((B, D), dtype=torch.float32, device=dev)
    de_dtype = torch.bfloat16 if args.de_dtype == "bf16" else torch.float32
    dE = torch.empty((M, D), dtype=de_dtype, device=dev)
    prof = genrec.Profiler(max_launches=80 * (args.steps + 1))

    def step(p=None):
        loss, lse, _ = genrec.ce_forward(H, E, lab, w, workspace=wsf, profiler=p)
        genrec.ce_backward(H, E, lab, lse, w, workspace=wsb, out=(dH, dE), profiler=p, de_dtype=de_dtype)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, med, mn = timed_steps(torch, step, args.steps)  # the timed steps, without the profiler
    ms_prof = timed_steps(torch, lambda: step(prof), args.steps)[0]  # per-kernel durations
    kern = prof.summary()
    per_step = {k: v[1] / args.steps for k, v in kern.items()}
    log("step %.3f ms; kernels per step %s" % (ms, {k: "%.3f ms" % v for k, v in per_step.items()}))
    # each MFMA kind computes one B x M x D product per step: 2 B M D flops
    prod = 2.0 * B * M * D
    tf = {k: prod / (per_step[k] * 1e-3) / 1e12 for k in ("main_score", "grad_tiles", "grad_E", "grad_H")
          if k in per_step}
    dom = max(tf, key=lambda k: per_step[k])
    kname = {"main_score": "mfma_score_kernel<1>", "grad_tiles": "mfma_score_kernel<3>",
             "grad_E": "mfma_score_kernel<4> (dE)", "grad_H": "mfma_score_kernel<4> (dH)"}[dom]
    res = {
        "metric": METRIC, "value": B * M / (ms * 1e-3), "unit": "scores/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": med,
        "ms_per_step_min": mn, "ms_per_step_profiled": ms_prof, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ce", "B": B, "D": D, "M": M, "step": "forward+backward",
                   "dE": args.de_dtype},
        "tflops": 4 * prod / (ms * 1e-3) / 1e12,
        "kernels_ms": per_step,
        "kernel_tflops": tf,
        "roofline": {"bound": "mfma", "achieved": tf[dom], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf[dom] / MFMA_BF16_PEAK_TFLOPS, "kernel": kname,
                     # one launch per catalog chunk: the mean launch, as the traffic figure
                     "kernel_ms": per_step[dom] * args.steps / kern[dom][0],
                     "launches_per_step": kern[dom][0] / args.steps,
                     # counters taken with the default fp32 dE
                     "traffic": traffic_from_profile({"grad_tiles": "mfma_score_kernel_3",
                                                      "grad_E": "mfma_score_kernel_4"}.get(dom, "none"), "ce")
                     if args.de_dtype == "f32" else None},
    }
    if not args.no_cpu_baseline:
        del H, E, dE, wsb
        torch.cuda.empty_cache()
        from oracle import oracle
        oracle.build()
        t0 = time.perf_counter()
        oracle.ce(d["H"], d["E"], d["labels"], d["weights"], users=[0])
        t1 = time.perf_counter() - t0
        n = int(max(1, min(B, args.cpu_seconds / max(t1, 1e-3))))
        users = np.linspace(0, B - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.ce(d["H"], d["E"], d["labels"], d["weights"], users=users)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = dict(value=n * M / t, unit="scores/s", cores=oracle.threads(), kind="oracle",
                                   sample="%d of %d users: loss, lse and dH rows (fp64; dE needs every user), "
                                          "%.1f s" % (n, B, t))
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    if args.peaks:
        peaks()
        return
    if args.workload.startswith("beam"):
        bench_beam(args)
        return
    if args.workload == "ce":
        bench_ce(args)
        return
    import torch
    from full_catalog_ranking_amd import genrec, synth

    dev = torch.device("cuda:0")
    genrec.lib()
    cfg = synth.WORKLOADS[args.workload]
    K = cfg["K"]
    t0 = time.perf_counter()
    if args.clusters and (args.workload in ("cand", "tiny") or cfg.get("kind")):
        raise SystemExit("--clusters applies to the full-catalog workloads")
    d = synth.make_workload(args.workload, **({"clusters": args.clusters} if args.clusters else {}))
    log("inputs generated in %.1f s" % (time.perf_counter() - t0))
    B, D, M = d["B"], d["D"], d["M"]
    H, E = to_dev(d["H"], dev, torch), to_dev(d["E"], dev, torch)
    cand = args.workload == "cand"
    if cand:
        off = torch.from_numpy(d["offsets"]).to(dev)
        ids = torch.from_numpy(d["ids"]).to(dev)
        nnz = int(d["ids"].size)
        ws = torch.empty(genrec.cand_workspace_bytes(B, D, M, nnz, K, H.dtype), dtype=torch.uint8, device=dev)
        units = nnz
    else:
        ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
        units = B * M
    out = (torch.empty((B, K), dtype=torch.int32, device=dev),
           torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B,), dtype=torch.float32, device=dev))
    prof = genrec.Profiler(max_launches=8 * (args.steps + 1))

    mask = None
    words = None
    if args.mask_density is not None:
        if cand:
            raise SystemExit("--mask-density applies to the full-catalog workloads")
        allowed = np.random.default_rng(12345).random(M) < args.mask_density
        W = (M + 31) // 32
        pad = np.zeros(W * 32, dtype=bool)
        pad[:M] = allowed
        words = (pad.reshape(W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
        mask = torch.from_numpy(words.view(np.int32)).to(dev)

    def step(p=None):
        if cand:
            genrec.score_candidates_topk(H, E, off, ids, K, workspace=ws, out=out, profiler=p)
        else:
            genrec.score_lse_topk(H, E, K, workspace=ws, out=out, profiler=p, mask=mask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    # timed region: the steps as a caller runs them; then the same steps again with
    # the library profiler's HIP events around every kernel (on the stream the
    # kernels run on) for the per-kernel durations -- those events add a few
    # microseconds to a step of a few short kernels, so they stay out of the
    # timed region
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()

    def cold_steps(p):
        # each step after a 1 GiB scratch write; only the steps are timed
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        per = []
        for _ in range(args.steps):
            scratch.fill_(1)
            start.record()
            step(p)
            end.record()
            torch.cuda.synchronize()
            per.append(start.elapsed_time(end))
        del scratch
        per.sort()
        med = per[args.steps // 2] if args.steps % 2 else 0.5 * (per[args.steps // 2 - 1] + per[args.steps // 2])
        return sum(per) / args.steps, med, per[0]

    if args.cold:
        ms, med, mn = cold_steps(None)
        ms_prof = cold_steps(prof)[0]
    elif args.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ms, med, mn = timed_steps(torch, g.replay, args.steps)
        del g
        ms_prof = timed_steps(torch, lambda: step(prof), args.steps)[0]  # per-kernel durations: eager steps
    else:
        ms, med, mn = timed_steps(torch, step, args.steps)
        ms_prof = timed_steps(torch, lambda: step(prof), args.steps)[0]
    kern = prof.summary()
    log("step %.3f ms; kernels %s" % (ms, {k: "%.3f ms x%d" % (v[1] / v[0], v[0]) for k, v in kern.items()}))
    rescued = None if cand else genrec.rescued_users(ws)  # of the last call

    n_main, t_main = kern["main_score"]
    main_ms = t_main / n_main
    flops = 2.0 * D * units
    if cand or not genrec.describe_plan(B, D, M, K, H.dtype)["path"] == "mfma":
        # VALU path over streamed / gathered rows: HBM-bound
        elem = 2 if H.dtype == torch.bfloat16 else 4
        if cand:
            uniq = np.unique(d["ids"]).size
            alg_bytes = uniq * D * elem + B * D * elem + nnz * 4 + (B + 1) * 8
        else:
            alg_bytes = M * D * elem + B * D * elem
        achieved = alg_bytes / (main_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=achieved / HBM_PEAK_GBS)
        # the same work over the whole call (every kernel of the step)
        roof["call_achieved"] = alg_bytes / (ms * 1e-3) / 1e9
        roof["call_frac"] = roof["call_achieved"] / HBM_PEAK_GBS
    else:
        peak = MFMA_BF16_PEAK_TFLOPS if H.dtype == torch.bfloat16 else FP32_MATRIX_PEAK_TFLOPS
        achieved = flops / (main_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=peak, unit="TFLOP/s", frac=achieved / peak)
        roof["call_achieved"] = flops / (ms * 1e-3) / 1e12
        roof["call_frac"] = roof["call_achieved"] / peak
    fused = not cand and genrec.describe_plan(B, D, M, K, H.dtype)["fused"] == 1
    roof["kernel"] = "mfma_score_kernel" if roof["bound"] == "mfma" else "stream_score_kernel"
    if fused:
        roof["kernel"] = "stream_score_kernel (fused: the whole call in one launch)"
    # the masked scoring kernel is its own instance: it has its own counter summary, if any
    roof["traffic"] = None if args.clusters else traffic_from_profile(
        roof["kernel"].split()[0], args.workload + ("_masked" if args.mask_density is not None else ""))
    roof["kernel_ms"] = main_ms

    res = {
        "metric": METRIC,
        "value": units / (ms * 1e-3),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": med,
        "ms_per_step_min": mn,
        "ms_per_step_profiled": ms_prof,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if H.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "D": D, "M": M, "K": K,
                   **({"nnz": units} if cand else {}), **({"cache": "cold"} if args.cold else {}),
                   **({"timing": "graph replay"} if args.graph and not args.cold else {}),
                   **({"mask_density": args.mask_density} if args.mask_density is not None else {}),
                   **({"catalog": "clustered", "clusters": args.clusters} if args.clusters else {})},
        "tflops": flops / (ms * 1e-3) / 1e12,
        "kernels_ms": {k: v[1] / v[0] for k, v in kern.items()},
        "roofline": roof,
    }
    if rescued is not None:
        res["rescued_users"] = rescued
    del H, E, ws
    torch.cuda.empty_cache()
    res["measured_peaks"] = peaks(emit=False)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, K, args.cpu_seconds, cand, words)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
