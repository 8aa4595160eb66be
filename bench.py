"""Merge-round throughput of the DiLoCo outer-step merge on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload KEY] [--no-cpu-baseline]

A step is one whole merge round of the workload (every fold of every
fragment, then every fragment's close), issued through the C ABI on inputs
already resident in HBM.  W untimed rounds, then K timed rounds between two
device synchronisations; every launch is bracketed by HIP events on the
stream it runs on, giving each kernel's average duration.  Prints one JSON
line: the HBM bytes the round moves per second, merged params/s, the
fraction of the 8 TB/s HBM peak, the workload's algorithmic bytes per second,
the roofline of the dominant kernel, the same round with each fragment's
arrivals passed in one call (`batched_round`, one pass per fragment), a plain
device-to-device copy as the box's reference point (`copy_ceiling`), and the
CPU oracle timed on a bounded sample of the same workload.

Default workload: DiffuRefill-1B (1,075,980,288 fp32 params) in 4 fragments,
5 fp32 workers, token-weighted delta mean + outer Nesterov (lr 0.7, momentum
0.9) + EMA (beta 0.9) fused per fragment.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
DEFAULT_WORKLOAD = "diffurefill1b_frag_nesterov_ema"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    from checkpoint_averaging_amd.profile_summary import kernel_source_hash as h
    return h()


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch of `kind` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    ks = d.get("kernels", {})
    # counter summaries name bf16-checkpoint kernels with a _bf16 suffix
    k = ks.get(kind) or ks.get(kind + "_bf16")
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def measured_dram_traffic(workload: str, kind: str):
    """DRAM bytes (read + write) per launch of `kind` from the committed
    summary of the raw request counters (no copy-kernel scale), if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"dram_traffic_{workload}_bench.json")
    if not os.path.exists(path):       # the benchmark's own process first, else the native driver
        path = os.path.join(ROOT, "profiles", f"dram_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(kind)
    if not k:
        return None
    return k["dram_read_bytes_per_launch"] + k["write_bytes_per_launch"]


def measured_polar_traffic(kind: str, batching: str):
    """HBM bytes per launch of an orthogonalisation kernel kind from the
    committed counter summary, if it was taken on the current source of the
    product kernels and with the same batching of the matrices (which sets
    the size of a launch); else None."""
    path = os.path.join(ROOT, "profiles", "pmc_diffurefill1b_orthogonal_step.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    from checkpoint_averaging_amd.profile_summary import polar_source_hash
    if d.get("kernel_source_hash") != polar_source_hash() or d.get("batching") != batching:
        return None
    k = d.get("kernels", {}).get(kind)
    return k.get("hbm_bytes_per_launch") if k else None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def cpu_baseline(w, torch, max_seconds: float = 12.0):
    """The oracle (unchanged) on a bounded sample of the workload: the first
    `per_frag` elements of every fragment, full round structure (every fold
    in arrival order, then the close).  Inputs are generated on the GPU by the
    seeded generator and copied to host memory before timing."""
    import numpy as np
    import oracle
    from checkpoint_averaging_amd import synth

    cores = len(os.sched_getaffinity(0))
    orc = oracle.load()
    orc.set_threads(cores)
    per_frag = min(1 << 24, min(w.frag_offsets[f + 1] - w.frag_offsets[f]
                                for f in range(w.n_frags)))
    n_s = per_frag * w.n_frags
    dev = torch.device("cuda")
    frags = []
    for f in range(w.n_frags):
        s = w.frag_offsets[f]
        th0 = synth.global0(w.seed, per_frag, device=dev, start=s)
        cks = []
        for i in range(w.workers):
            c = synth.worker_checkpoint(w.seed, 0, i, th0, start=s, dtype=w.ckpt_dtype)
            c = c.cpu()
            cks.append(c.view(torch.int16).numpy().view(np.uint16).copy()
                       if w.ckpt_dtype == "bf16" else c.numpy().copy())
        th = th0.cpu().numpy().copy()
        frags.append({"theta": th, "m": np.zeros_like(th), "e": th.copy() if w.ema else None,
                      "cks": cks})
    orders = [synth.arrival_order(w, 0, f) for f in range(w.n_frags)]
    tok = synth.token_counts(w, 0)
    from checkpoint_averaging_amd.workload import algorithmic_bytes
    bytes_per_round = algorithmic_bytes(w)["per_param"] * n_s

    def time_rounds(limit):
        rounds = 0
        t0 = time.perf_counter()
        while True:
            for f, F in enumerate(frags):
                order = orders[f]
                if w.mode == "mean":
                    F["theta"] = orc.mean_round([F["cks"][i] for i in order], ema=F["e"],
                                                beta=w.beta)
                else:
                    orc.nesterov_fragment_round(F["theta"], F["m"],
                                                [F["cks"][i] for i in order],
                                                [tok[i] for i in order], w.lr, w.mu, F["e"],
                                                w.beta)
            rounds += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return rounds, el

    rounds, el = time_rounds(max_seconds)
    sec = el / rounds
    out = {
        "value": round(bytes_per_round / sec / 1e9, 3), "unit": "GB/s",
        "params_per_s": round(n_s / sec, 1),
        "cores": orc.threads(), "kind": "oracle",
        "sample": (f"first {per_frag:,} elements of each of the {w.n_frags} fragment(s) "
                   f"({n_s:,} params, {w.workers} {w.ckpt_dtype} workers), full round "
                   f"structure, {rounds} rounds in {el:.1f} s"),
        "cpu": cpu_model(),
    }
    if w.n_params < (1 << 26):
        # the small (Pythia-14M) workloads are also timed on one thread
        orc.set_threads(1)
        r1, el1 = time_rounds(max_seconds / 2)
        orc.set_threads(cores)
        sec1 = el1 / r1
        out["single_core"] = {"value": round(bytes_per_round / sec1 / 1e9, 3), "unit": "GB/s",
                              "params_per_s": round(n_s / sec1, 1), "cores": 1,
                              "sample": f"{r1} rounds in {el1:.1f} s"}
    return out


# kind (as the counter summaries name it) of each product kernel
POLAR_KIND = {"k_gemm_big<NT>": "gemm_big_NT", "k_gemm_big<TN>": "gemm_big_TN",
              "k_gemm<NT>": "gemm_NT", "k_gemm<TN>": "gemm_TN"}

# kernel kind (as the counter summaries name it) of each side-average call
SIDE_KERNEL_KIND = {"swa_fold": "fold", "swa_average": "finalize_mean",
                    "snapshot_average_3": "snapshot_mean_3",
                    "snapshot_average_5": "snapshot_mean_5", "adopt_keep_drift": "adopt_keep_drift"}


def side_averages(args, torch):
    """Times the side averages at the DiffuRefill-1B size: folding a global
    into the uniform-average sum (12 B/param), the average itself
    (8 B/param), the one-pass averages of the last 3 and last 5 snapshots
    (16 and 24 B/param), and the worker-side keep-local-drift adoption
    (16 B/param).  One JSON line."""
    from checkpoint_averaging_amd import dlmerge as dl
    from checkpoint_averaging_amd import synth
    n = synth.DIFFUREFILL_1B.n_params
    dev = torch.device("cuda")
    th0 = synth.global0(1006, n, device=dev)
    snaps = [synth.worker_checkpoint(1006, r, 0, th0) for r in range(5)]
    del th0
    acc = torch.empty(n, device=dev)
    out = torch.empty(n, device=dev)
    torch.cuda.synchronize()
    cases = {
        "swa_fold": (12, lambda i: dl.dl_swa_fold(acc, snaps[i % 5], 1 + i)),
        "swa_average": (8, lambda i: dl.dl_swa_average(out, acc, 130)),
        "snapshot_average_3": (16, lambda i: dl.dl_snapshot_average(out, snaps[:3])),
        "snapshot_average_5": (24, lambda i: dl.dl_snapshot_average(out, snaps)),
        # worker-side keep-local-drift adoption: theta += global - pushed
        "adopt_keep_drift": (16, lambda i: dl.dl_adopt_keep_drift(out, snaps[0], snaps[1])),
    }
    res = {}
    for name, (bpe, call) in cases.items():
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        evs = []
        for i in range(args.steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            call(i)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        res[name] = {"avg_ms": round(ms, 4), "bytes_per_param": bpe,
                     "GB_per_s": round(bpe * n / (ms / 1e3) / 1e9, 1),
                     "frac_of_hbm_peak": round(bpe * n / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] {name}: {ms:.3f} ms")
    # the dominant call: the longest per launch (all run the same count)
    dom = max(res, key=lambda k: res[k]["avg_ms"])
    dd = res[dom]
    achieved = dd["bytes_per_param"] * n / (dd["avg_ms"] / 1e3) / 1e9
    out_line = {
        "metric": "side averages of the globals and worker adoption: effective HBM GB/s",
        "value": dd["GB_per_s"], "unit": "GB/s", "n_gpus": 1,
        "n_params": n, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "dtype": "f32", "data": "synthetic (seeded Philox; DiffuRefill-1B size)",
        "config": {"workload": "diffurefill1b_side_averages", "n_params": n},
        "kernels": res,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("diffurefill1b_side_averages",
                                                 SIDE_KERNEL_KIND[dom]),
                     "algorithmic_bytes_per_launch": dd["bytes_per_param"] * n},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del acc, out, snaps
        torch.cuda.empty_cache()
        out_line["cpu_baseline"] = cpu_baseline_side(dom)
    print(json.dumps(out_line), flush=True)


def cpu_baseline_side(dom: str, max_seconds: float = 3.0):
    """The unchanged oracle's side averages and adoption on 16,777,216
    elements each, repeated for about max_seconds per call; effective GB/s
    per call (same bytes per param as on the GPU)."""
    import numpy as np
    import oracle
    n = 1 << 24
    rng = np.random.default_rng(1006)
    snaps = [rng.standard_normal(n).astype(np.float32) * np.float32(0.02) for _ in range(5)]
    acc = np.empty(n, np.float32)
    outb = np.empty(n, np.float32)
    orc = oracle.load()
    cases = {
        "swa_fold": (12, lambda: orc.fold_mean(acc, snaps[1], first=False)),
        "swa_average": (8, lambda: orc.finalize_mean(outb, acc, 130)),
        "snapshot_average_3": (16, lambda: orc.snapshot_average(snaps[:3])),
        "snapshot_average_5": (24, lambda: orc.snapshot_average(snaps)),
        "adopt_keep_drift": (16, lambda: orc.adopt_keep_drift(outb, snaps[0], snaps[1])),
    }
    orc.fold_mean(acc, snaps[0], first=True)
    per = {}
    for name, (bpe, call) in cases.items():
        call()                                   # first touch of the output pages
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < max_seconds:
            call()
            done += 1
        el = time.perf_counter() - t0
        per[name] = round(bpe * n * done / el / 1e9, 2)
    return {"value": per[dom], "unit": "GB/s", "cores": orc.threads(), "kind": "oracle",
            "per_call_GB_per_s": per,
            "sample": f"16,777,216 elements per call, each call repeated for ~{max_seconds:.0f} s "
                      f"on {cpu_model()}"}


MFMA_F32_PEAK_TFLOPS = 157.3


def orthogonalize(args, torch):
    """Times one orthogonalised outer step over every DiffuRefill-1B weight
    matrix (theta = theta - s * P(theta - averaged), P the polar factor by 12
    quintic + 6 cubic Newton-Schulz steps), matrix by matrix on one stream,
    and every distinct fp32 MFMA product of the iteration launch by launch.
    One JSON line."""
    import numpy as np
    from checkpoint_averaging_amd import dlmerge as dl
    from checkpoint_averaging_amd import synth
    from checkpoint_averaging_amd.orthogonalize import OrthogonalStep, gemm_flops, product_kernel

    layout = synth.DIFFUREFILL_1B
    dev = torch.device("cuda")
    n = layout.n_params
    theta = synth.global0(1007, n, device=dev)
    averaged = synth.worker_checkpoint(1007, 0, 0, theta)
    step = OrthogonalStep(layout, dev, batch=args.orth_batch or None, streams=args.orth_streams)
    mats = step.matrices
    n_mat = sum(m.rows * m.cols for m in mats)
    flops = step.flops()
    scale = 1e-4
    torch.cuda.synchronize()
    log(f"[bench] orthogonalise: {len(mats)} matrices, {n_mat:,} params, "
        f"{sum(flops.values()) / 1e12:.1f} TFLOP per step")
    for _ in range(args.warmup):
        step.run(theta, averaged, scale)
    torch.cuda.synchronize()
    recs = []

    def timer(g, call):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        recs.append((g, e0, e1))

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(theta, averaged, scale, timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    by_shape = {}
    for g, e0, e1 in recs:
        d = by_shape.setdefault((g[0].rows, g[0].cols), [0, 0.0])
        d[0] += len(g)
        d[1] += e0.elapsed_time(e1)
    shapes = {}
    for (r, c), (cnt, tot) in by_shape.items():
        f = sum(gemm_flops(r, c).values())
        shapes[f"{r}x{c}"] = {"matrices_per_step": cnt // args.steps,
                              "avg_ms_per_matrix": round(tot / cnt, 3),
                              "TFLOP_per_s": round(f / (tot / cnt / 1e3) / 1e12, 2)}
    log(f"[bench] {args.steps} orthogonalised steps: {ms:.1f} ms/step")

    # every distinct product of the iteration, timed launch by launch through
    # the same kernels with the same launch shapes: per batch of equally
    # shaped matrices, the symmetric Gram product, its symmetric square and
    # the next iterate, with a workspace for the stream-K split (values: an
    # iterate-like X and a symmetric Gram-like G)
    import collections
    gcount = collections.Counter((g[0].rows, g[0].cols, len(g)) for g in step.groups)
    prods = {}
    for (r_, c_, bsz), ngroups in gcount.items():
        r, L = min(r_, c_), max(r_, c_)
        tall = r_ >= c_
        sx, sg = r_ * c_, r * r
        x = torch.randn(bsz * sx, device=dev).mul_(1.0 / np.sqrt(L))
        g = torch.randn(bsz, r, r, device=dev).mul_(1.0 / r)
        g = (g + g.transpose(1, 2)).contiguous().view(-1)                  # symmetric
        out_x = torch.empty(bsz * sx, device=dev)
        out_g = torch.empty(bsz * sg, device=dev)
        if tall:
            cases = [("TN", "gram", (x, c_, sx, x, c_, sx, r, r, L, out_g, r, sg), True, 18),
                     ("NT", "gram_square", (g, r, sg, g, r, sg, r, r, r, out_g, r, sg), True, 12),
                     ("NT", "next_iterate", (x, c_, sx, g, r, sg, L, r, r, out_x, c_, sx), False,
                      18)]
        else:
            cases = [("NT", "gram", (x, c_, sx, x, c_, sx, r, r, L, out_g, r, sg), True, 18),
                     ("NT", "gram_square", (g, r, sg, g, r, sg, r, r, r, out_g, r, sg), True, 12),
                     ("TN", "next_iterate", (g, r, sg, x, c_, sx, r, L, r, out_x, c_, sx), False,
                      18)]
        for form, what, a, sym, per in cases:
            fm = dl.DL_TN if form == "TN" else dl.DL_NT
            M, N, K = a[6], a[7], a[8]
            wsb = dl.dl_matmul_workspace_bytes_batch(M, N, K, sym, bsz)
            ws = torch.empty(max(wsb, 256) // 4, dtype=torch.float32, device=dev)
            call = lambda fm=fm, a=a, sym=sym, ws=ws, bsz=bsz: dl.dl_matmul_f32_batch(
                fm, *a, bsz, symmetric=sym, workspace=ws)
            call()
            torch.cuda.synchronize()
            evs = []
            for _ in range(max(3, args.steps)):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
            avg = sum(p.elapsed_time(q) for p, q in evs) / len(evs)
            outs = M * (M + 1) // 2 if sym else M * N      # distinct outputs
            fl = 2 * outs * K * bsz
            prods[f"{form} {what} {M}x{N}x{K} batch {bsz} of {r_}x{c_}"] = {
                "form": form, "kernel": product_kernel(form, M, N, K, bsz, sym),
                "symmetric": sym, "batch": bsz, "launches_per_step": per * ngroups,
                "avg_ms": round(avg, 4), "flops_per_launch": fl,
                "TFLOP_per_s": round(fl / (avg / 1e3) / 1e12, 2)}
            del ws
        del x, g, out_x, out_g
    kinds = {}
    for p in prods.values():
        d = kinds.setdefault(p["kernel"], {"ms": 0.0, "flops": 0, "launches": 0})
        d["ms"] += p["avg_ms"] * p["launches_per_step"]
        d["flops"] += p["flops_per_launch"] * p["launches_per_step"]
        d["launches"] += p["launches_per_step"]
    dom = max(kinds, key=lambda k: kinds[k]["ms"])
    dd = kinds[dom]
    achieved = dd["flops"] / (dd["ms"] / 1e3) / 1e12
    total_flops = sum(flops.values())
    out = {
        "metric": "orthogonalised outer step over every DiffuRefill-1B weight matrix: "
                  "matrix params/s",
        "value": round(n_mat / (ms / 1e3), 1),
        "unit": "params/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 2),
        "higher_is_better": True,
        "dtype": "f32",
        "data": "synthetic (seeded Philox; DiffuRefill-1B matrix shapes)",
        "config": {"workload": "diffurefill1b_orthogonal_step", "matrices": len(mats),
                   "batch": (args.orth_batch or
                             "each shape's matrices together, split evenly into launches of "
                             "at most 64"),
                   "batches": sorted({f"{len(g)} x {g[0].rows}x{g[0].cols}"
                                      for g in step.groups}),
                   "streams": args.orth_streams,
                   "matrix_params": n_mat, "quintic_steps": 12, "cubic_steps": 6,
                   "algorithmic_flops_per_step": total_flops},
        "TFLOP_per_s": round(total_flops / (ms / 1e3) / 1e12, 2),
        "frac_of_mfma_f32_peak": round(total_flops / (ms / 1e3) / 1e12 / MFMA_F32_PEAK_TFLOPS, 4),
        "shapes": shapes,
        "products": prods,
        "roofline": {"kernel": dom, "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F32_PEAK_TFLOPS, 4),
                     "traffic": measured_polar_traffic(POLAR_KIND[dom],
                                                       str(args.orth_batch or "even")),
                     "algorithmic_flops_per_launch": dd["flops"] // dd["launches"],
                     "avg_launch_ms": round(dd["ms"] / dd["launches"], 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del theta, averaged, step
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline_polar()
    print(json.dumps(out), flush=True)


def cpu_baseline_polar(max_seconds: float = 12.0):
    """The orthogonalisation oracle (fp64 SVD polar factor, unchanged) on
    2048 x 2048 attention-shaped updates until about max_seconds have
    passed; matrix params per second."""
    import numpy as np
    from oracle import polar
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:       # threadpoolctl missing: report the CPU count numpy may use
        cores = os.cpu_count() or 1
    rng = np.random.default_rng(1007)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < max_seconds:
        a = (rng.standard_normal((2048, 2048)) * 1e-3).astype(np.float32)
        polar.polar_factor(a)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(done * 2048 * 2048 / el, 1), "unit": "params/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} updates of 2048x2048 (one attention matrix each), fp64 SVD polar "
                      f"factor, {el:.1f} s on {cpu_model()}"}


def copy_ceiling(torch, nbytes: int = 4 << 30, reps: int = 5):
    """Plain device-to-device copies of nbytes, timed with events (read +
    write bytes per second), as the box's reference point for the streaming
    kernels: the library's own engine copying (dl_swa_fold with nothing
    folded before is sum = global, one pack per lane, non-temporal), and
    torch's copy_."""
    from checkpoint_averaging_amd import dlmerge as dl
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)

    def median_ms(call):
        call()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]

    eng = median_ms(lambda: dl.dl_swa_fold(dst, src, 0))
    tch = median_ms(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    gbs = lambda ms: 2 * nbytes / (ms / 1e3) / 1e9
    return {"engine_copy_GB_per_s": round(gbs(eng), 1),
            "engine_copy_frac_of_hbm_peak": round(gbs(eng) / HBM_PEAK_GBS, 4),
            "torch_copy_GB_per_s": round(gbs(tch), 1),
            "bytes_each_way": nbytes,
            "method": ("median of %d copies each: the library's streaming engine "
                       "(dl_swa_fold with nothing folded before), and torch copy_" % reps)}


def batched_round(gw, w, ab, args, torch):
    """The same round with every fragment's arrivals passed in one
    several-arrival call that also closes (all checkpoints are resident): one
    pass per fragment.  Same buffers, same results bit for bit; W untimed and
    K timed rounds, each launch between events on its stream."""
    for r in range(args.warmup):
        gw.run_round(0, tag=7000 + r, batched=True)
    torch.cuda.synchronize()
    records, spans = [], []

    def timed(kind, n, call):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        records.append((kind, n, e0, e1))

    t0 = time.perf_counter()
    for r in range(args.steps):
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        r0.record()
        gw.run_round(0, tag=8000 + r, timer=timed, batched=True)
        r1.record()
        spans.append((r0, r1))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"[bench] {args.steps} timed batched rounds: {ms:.3f} ms/round")
    per = sorted(a.elapsed_time(b) for a, b in spans)
    kind = records[0][0]
    launches = len(records)
    kms = sum(e0.elapsed_time(e1) for _, _, e0, e1 in records)
    kbytes = sum(ab["per_elem"][k] * n for k, n, _, _ in records)
    achieved = kbytes / (kms / 1e3) / 1e9
    moved = ab["per_round_batched"]
    value = moved / (ms / 1e3) / 1e9
    return {
        "round_schedule": ("every arrival of a fragment passed in one call, in arrival order: "
                           "one pass per fragment folds them all and closes"),
        "ms_per_step": round(ms, 4),
        "round_ms_median": round(per[len(per) // 2], 4),
        "moved_bytes_per_param": ab["per_param_batched"],
        "moved_GB_per_s": round(value, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "merged_params_per_s": round(w.n_params / (ms / 1e3), 1),
        "speedup_vs_per_arrival_round": None,
        "roofline": {
            "kernel": kind,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.key, kind),
            "traffic_raw_dram_counters": measured_dram_traffic(w.key, kind),
            "algorithmic_bytes_per_launch": kbytes // launches,
            "avg_ms": round(kms / launches, 4),
        },
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-close", action="store_true",
                    help="close each fragment in its own pass after the last fold, instead of "
                         "folding the last arrival into the close")
    ap.add_argument("--batched", action="store_true",
                    help="pass each fragment's arrivals to the library in one several-arrival "
                         "call (every checkpoint resident): one pass per fragment")
    ap.add_argument("--graph", action="store_true",
                    help="capture one round into a HIP graph and time its replays (the "
                         "per-kernel figures still come from event-timed eager rounds)")
    ap.add_argument("--fragment-streams", type=int, default=0,
                    help="run every fragment's round as its own handle on one of this many "
                         "streams (rounds in flight together)")
    ap.add_argument("--side-averages", action="store_true",
                    help="time the uniform average and snapshot averages instead of a round")
    ap.add_argument("--orthogonalize", action="store_true",
                    help="time the orthogonalised outer step over every weight matrix instead "
                         "of a merge round")
    ap.add_argument("--orth-batch", type=int, default=0,
                    help="equally shaped matrices orthogonalised together (1: one by one; "
                         "0: all of a shape, split evenly into launches of at most 64)")
    ap.add_argument("--orth-streams", type=int, default=1,
                    help="streams the orthogonalised step's batches are spread over")
    ap.add_argument("--runtime-fill", action="store_true",
                    help="fill the inputs with constants through the HIP runtime's memset "
                         "instead of the seeded generator, so that the process launches no "
                         "torch kernel (for counter runs under the profiler; timing and "
                         "traffic do not depend on the values)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB "
                         "(for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the merge shards with no exchange step; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from checkpoint_averaging_amd import synth
    from checkpoint_averaging_amd.workload import GpuWorkload, algorithmic_bytes

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.side_averages:
        side_averages(args, torch)
        return
    if args.orthogonalize:
        orthogonalize(args, torch)
        return
    w = synth.WORKLOADS[args.workload]
    ab = algorithmic_bytes(w)
    log(f"[bench] {w.key}: {w.n_params:,} params, {w.workers} {w.ckpt_dtype} workers, "
        f"{w.n_frags} fragment(s), {ab['per_param']} B/param")
    if args.runtime_fill and args.copy_calibration_mib:
        sys.exit("--copy-calibration-mib runs torch kernels; it does not combine with "
                 "--runtime-fill")
    gw = GpuWorkload(w, fill="runtime" if args.runtime_fill else "philox")
    gw.generate_checkpoints(0)
    torch.cuda.synchronize()
    log("[bench] inputs resident")

    if args.copy_calibration_mib:
        # one elementwise kernel that reads nb bytes and writes nb bytes
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: elementwise kernel, {nb} bytes read, {nb} bytes written")
        del src, dst

    def plain(kind, n, call):
        call()

    fused = not args.separate_close
    streams = ([torch.cuda.Stream() for _ in range(args.fragment_streams)]
               if args.fragment_streams > 0 else None)
    for r in range(args.warmup):
        gw.run_round(0, tag=r + 1, timer=plain, fused_close=fused, streams=streams,
                     batched=args.batched)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup rounds done")

    records = []

    def timed(kind, n, call):
        # events on the stream the call launches on (torch's current stream,
        # which the binding passes to the library)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        records.append((kind, n, e0, e1))

    spans = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(args.steps):
        if streams is None:
            # each round's span on the stream, first launch to last
            r0 = torch.cuda.Event(enable_timing=True)
            r1 = torch.cuda.Event(enable_timing=True)
            r0.record()
        gw.run_round(0, tag=1000 + r, timer=timed if streams is None else plain,
                     fused_close=fused, streams=streams, batched=args.batched)
        if streams is None:
            r1.record()
            spans.append((r0, r1))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    log(f"[bench] {args.steps} timed rounds: {ms:.3f} ms/round")
    graph = None
    if args.graph:
        if streams is not None:
            sys.exit("--graph captures one stream; it does not combine with --fragment-streams")
        # capture records the round's launches without running them; every
        # replay then runs the same folds and close on the same buffers
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gw.run_round(0, tag=5000, timer=plain, fused_close=fused, batched=args.batched)
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        log(f"[bench] {args.steps} graph replays: {gms:.3f} ms/round")
        graph = {"ms_per_round": round(gms, 4), "eager_ms_per_round": round(ms, 4)}
        ms = gms
    round_ms = None
    if spans:
        per = sorted(a.elapsed_time(b) for a, b in spans)
        mid = len(per) // 2
        med = per[mid] if len(per) % 2 else 0.5 * (per[mid - 1] + per[mid])
        round_ms = {"median": round(med, 4), "min": round(per[0], 4), "max": round(per[-1], 4),
                    "basis": "stream events around each timed round"}

    kinds = {}
    for kind, n, e0, e1 in records:
        d = kinds.setdefault(kind, {"launches": 0, "ms": 0.0, "bytes": 0})
        d["launches"] += 1
        d["ms"] += e0.elapsed_time(e1)
        d["bytes"] += ab["per_elem"][kind] * n
    kern = {}
    for kind, d in kinds.items():
        kern[kind] = {"launches_per_round": d["launches"] // args.steps,
                      "avg_ms": round(d["ms"] / d["launches"], 4),
                      "GB_per_s": round(d["bytes"] / (d["ms"] / 1e3) / 1e9, 1),
                      "share_of_kernel_time": None}
    total_kernel_ms = sum(d["ms"] for d in kinds.values())
    for kind, d in kinds.items():
        kern[kind]["share_of_kernel_time"] = round(d["ms"] / total_kernel_ms, 3)
    roofline = None
    if kinds:
        dom = max(kinds, key=lambda k: kinds[k]["ms"])
        dd = kinds[dom]
        achieved = dd["bytes"] / (dd["ms"] / 1e3) / 1e9
        roofline = {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.key, dom),
            "traffic_raw_dram_counters": measured_dram_traffic(w.key, dom),
            "algorithmic_bytes_per_launch": dd["bytes"] // dd["launches"],
        }
    # value: the HBM bytes the timed schedule moves per round / round time.
    # The algorithmic bytes of the separate-close schedule (every arrival
    # folded, then the close) are reported beside it: the fused close moves
    # fewer bytes for the same round, so dividing those by its time would
    # credit bytes it never streams.
    if args.batched:
        moved = ab["per_round_batched"] if fused else ab["per_round_batched_separate"]
    else:
        moved = ab["per_round_fused"] if fused else ab["per_round"]
    value = moved / (ms / 1e3) / 1e9
    algorithmic = ab["per_round"] / (ms / 1e3) / 1e9
    if args.batched:
        schedule = ("every arrival of a fragment passed in one call, in arrival order: "
                    + ("one pass per fragment folds them all and closes" if fused else
                       "one pass folds them all, the close a separate pass"))
    else:
        schedule = ("each arrival folded on its own; the last arrival of each fragment folded "
                    "in the same pass as the close" if fused else
                    "each arrival folded on its own; the close a separate pass")
    out = {
        "metric": "merge-round throughput: effective HBM GB/s and merged params/s; % of HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": ("synthetic (constants from the HIP runtime's memset; counter run)"
                 if args.runtime_fill else
                 "synthetic (seeded Philox; shapes of the pages' models)"),
        "config": {
            "workload": w.key,
            "description": w.description,
            "n_params": w.n_params,
            "workers": w.workers,
            "checkpoint_dtype": w.ckpt_dtype,
            "fragments": w.n_frags,
            "algorithmic_bytes_per_param": ab["per_param"],
            "algorithmic_bytes_per_round": ab["per_round"],
            "round_schedule": schedule,
        },
        "value_basis": ("HBM bytes the timed schedule moves per round (each buffer a pass "
                        "touches counted once per pass) / round time"),
        "moved_bytes_per_param": moved // w.n_params,
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "merged_params_per_s": round(w.n_params / (ms / 1e3), 1),
        "algorithmic_bytes_per_param": ab["per_param"],
        "algorithmic_GB_per_s": round(algorithmic, 1),
        "algorithmic_frac_of_hbm_peak": round(algorithmic / HBM_PEAK_GBS, 4),
        "algorithmic_basis": ("bytes of the per-arrival round with a separate close (every "
                              "arrival folded and written back, then every state buffer read "
                              "and written once) / round time; schedules that fuse passes "
                              "move fewer bytes (value), so this can exceed what HBM streams"),
        "kernel_time_ms_per_step": (round(total_kernel_ms / args.steps, 4) if kinds else None),
        "round_ms": round_ms,
        "graph": graph,
        "fragment_streams": args.fragment_streams,
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": None,
        "copy_ceiling": None,
    }
    if not args.batched and streams is None and not args.graph and args.steps > 0:
        out["batched_round"] = batched_round(gw, w, ab, args, torch)
        out["batched_round"]["speedup_vs_per_arrival_round"] = round(
            ms / out["batched_round"]["ms_per_step"], 3)
    if not args.runtime_fill and w.n_params >= (1 << 28):
        out["copy_ceiling"] = copy_ceiling(torch)
        log(f"[bench] plain copy: {out['copy_ceiling']['engine_copy_GB_per_s']} GB/s "
            f"(library engine), {out['copy_ceiling']['torch_copy_GB_per_s']} GB/s (torch)")
    if not args.no_cpu_baseline:
        del gw
        torch.cuda.empty_cache()
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
