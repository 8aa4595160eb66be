"""Summaries of rocprofv3 output for the merge kernels and the
orthogonalisation kernels.

    python -m checkpoint_averaging_amd.profile_summary stats STATS_CSV --command CMD
        -> markdown table of the merge kernels' dispatch durations
    python -m checkpoint_averaging_amd.profile_summary pmc FETCH_CSV WRITE_CSV \
        --workload KEY --command-fetch CMD --command-write CMD [--json OUT]
        -> HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE, each scaled by
           what the same counter reads for the plain copy kernel of known size

    python -m checkpoint_averaging_amd.profile_summary pmc-dram READ_CSV WRITE_CSV \
        --workload KEY --command-read CMD --command-write CMD [--json OUT]
        -> DRAM read bytes from the 32-byte-unit request counter and write bytes
           from the write requests, per dispatch, with no calibration

    python -m checkpoint_averaging_amd.profile_summary polar-stats STATS_CSV --command CMD
    python -m checkpoint_averaging_amd.profile_summary polar-pmc RUN_DIR --command CMD \
        --copy-bytes B [--json OUT]
        -> the same for the orthogonalisation kernels; RUN_DIR holds one
           rocprofv3 --pmc output directory per pass (FETCH_SIZE, WRITE_SIZE,
           TCC_HIT_sum, SQ_VALU_MFMA_BUSY_CYCLES), each from the same command

Kernel kinds follow the names the benchmark uses (fold, fold_first,
fold_delta, fold_delta_first, finalize_mean[_ema], nesterov[_ema],
fold_finalize_mean[_ema][_first], fold_nesterov[_ema][_first], ema,
snapshot_mean_K, adopt_keep_drift; for several arrivals in one pass
fold_all, fold_delta_all, fold_all_finalize_mean[_ema],
fold_all_nesterov[_ema], with _more when earlier folds came first; _bf16 for
bf16 checkpoints).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_kind(name: str):
    """Benchmark kind of a merge kernel from its demangled name, or None.

    Kernels are k_stream<Op, NT> (128-bit path) or k_stream_scalar<Op>; the
    kind comes from the operation and its template arguments."""
    m = re.search(r"::(FoldManyMeanClose|FoldManyNesterovClose|FoldSumMany|FoldDeltaMany|"
                  r"FoldMeanClose|FoldNesterovClose|FoldSum|FoldDelta|MeanClose|"
                  r"NesterovClose|Ema|SnapshotMean|AdoptKeepDrift)\b(?:<([^>]*)>)?", name)
    if not m or "k_stream" not in name:
        return None
    op = m.group(1)
    targs = [t.strip() for t in (m.group(2) or "").split(",")]
    if op == "SnapshotMean":
        return f"snapshot_mean_{targs[0]}"
    if op == "AdoptKeepDrift":
        return "adopt_keep_drift" + ("_bf16" if "short" in targs[0] else "")
    bf16 = "_bf16" if targs and "short" in targs[0] else ""
    # several arrivals in one pass: the kinds of a call holding every arrival
    # of the fragment (nothing folded before it); "_more" after earlier folds
    more = "" if len(targs) > 1 and targs[1] == "true" else "_more"
    if op == "FoldSumMany":
        return "fold_all" + more + bf16
    if op == "FoldDeltaMany":
        return "fold_delta_all" + more + bf16
    if op in ("FoldManyMeanClose", "FoldManyNesterovClose"):
        base = "fold_all_finalize_mean" if op == "FoldManyMeanClose" else "fold_all_nesterov"
        return base + ("_ema" if targs[2] == "true" else "") + more + bf16
    if op == "FoldSum":
        return ("fold_first" if targs[1] == "true" else "fold") + bf16
    if op == "FoldDelta":
        return ("fold_delta_first" if targs[1] == "true" else "fold_delta") + bf16
    if op == "MeanClose":
        return "finalize_mean_ema" if targs[0] == "true" else "finalize_mean"
    if op == "NesterovClose":
        return "nesterov_ema" if targs[0] == "true" else "nesterov"
    if op in ("FoldMeanClose", "FoldNesterovClose"):
        base = "fold_finalize_mean" if op == "FoldMeanClose" else "fold_nesterov"
        return (base + ("_ema" if targs[2] == "true" else "")
                + ("_first" if targs[1] == "true" else "") + bf16)
    return "ema"


# The side averages and the worker adoption, counted on dlmerge_driver --side 1:
# algorithmic bytes per element of each kernel kind (the uniform-average fold
# reads the sum and the global and writes the sum; the first fold only copies;
# the average reads the sum and writes the result; the k-snapshot mean reads k
# buffers and writes one; the adoption reads theta, the global and the pushed
# checkpoint and writes theta).
SIDE_WORKLOAD = "diffurefill1b_side_averages"
SIDE_BYTES_PER_ELEM = {"fold": 12, "fold_first": 8, "finalize_mean": 8, "snapshot_mean_3": 16,
                       "snapshot_mean_5": 24, "adopt_keep_drift": 16}


def strip_comments(src: str) -> str:
    """C/C++ source without its comments (string and character literals kept)
    and with runs of whitespace collapsed: what the compiler sees."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(*names: str) -> str:
    """Hash of the given csrc files' code (comments and layout ignored), so
    that counter summaries stay valid across comment edits and go stale
    with any change to the code itself."""
    h = hashlib.sha256()
    for f in names:
        with open(os.path.join(ROOT, "checkpoint_averaging_amd", "csrc", f)) as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash("kernels.hip", "kernels.h")


def polar_kind(name: str):
    """Kind of an orthogonalisation kernel from its demangled name, or None."""
    if "k_gemm<true>" in name:
        return "gemm_TN"
    if "k_gemm<false>" in name:
        return "gemm_NT"
    if "k_gemm_big<true>" in name:
        return "gemm_big_TN"
    if "k_gemm_big<false>" in name:
        return "gemm_big_NT"
    for k in ("k_reduce_pieces", "k_reduce_splits", "k_reduce_big", "k_sumsq_partial",
              "k_sumsq_final", "k_scale", "k_step"):
        if f"::{k}(" in name or name.startswith(k + "("):
            return k[2:]
    return None


def polar_source_hash() -> str:
    return source_hash("polar.hip", "polar.h")


def polar_stats_markdown(stats_csv: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["# Orthogonalisation kernels: dispatch durations (rocprofv3 --kernel-trace --stats)",
           "", "Command:", "", "```", command, "```", "",
           "| kind | calls | average (us) | min (us) | max (us) | total (ms) |",
           "|---|---:|---:|---:|---:|---:|"]
    other_calls, other_ns = 0, 0.0
    for r in rows:
        kind = polar_kind(r["Name"])
        calls, total = int(r["Calls"]), float(r["TotalDurationNs"])
        if kind is None:
            other_calls += calls
            other_ns += total
            continue
        out.append(f"| {kind} | {calls} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{total / 1e6:.2f} |")
    out += ["", f"Other kernels in the same run (input generation, torch): {other_calls} "
            f"dispatches, {other_ns / 1e6:.1f} ms in total.", ""]
    return "\n".join(out)


def polar_pmc_summary(run_dir: str, command: str, copy_bytes: int,
                      batching: str = "even") -> dict:
    """Per-kind sums over one pass per counter group, FETCH_SIZE / WRITE_SIZE
    scaled by the plain copy of known size; MFMA busy as a fraction of SIMD
    cycles (GRBM_GUI_ACTIVE counts per XCD: the max over the 8 is the
    dispatch's active cycles, here taken as the sum / 8); L2 hit rate."""
    def rows(tag):
        path = os.path.join(run_dir, tag, "run_counter_collection.csv")
        return list(csv.DictReader(open(path))) if os.path.exists(path) else []

    acc = defaultdict(lambda: defaultdict(float))
    launches = defaultdict(set)
    scale = {}
    for tag, counters in (("FETCH_SIZE", ("FETCH_SIZE",)), ("WRITE_SIZE", ("WRITE_SIZE",)),
                          ("TCC_HIT_sum", ("TCC_HIT_sum", "TCC_MISS_sum")),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", ("SQ_VALU_MFMA_BUSY_CYCLES",
                                                       "GRBM_GUI_ACTIVE",
                                                       "SQ_INSTS_VALU_MFMA_MOPS_F32"))):
        rs = rows(tag)
        for c in counters:
            if c in ("FETCH_SIZE", "WRITE_SIZE"):
                cp = [r for r in rs if "plain_copy" in r["Kernel_Name"] and r["Counter_Name"] == c]
                if len(cp) != 1:
                    raise SystemExit(f"{tag}: expected exactly one plain_copy dispatch")
                scale[c] = copy_bytes / (float(cp[0]["Counter_Value"]) * 1024)
        for r in rs:
            kind = polar_kind(r["Kernel_Name"].replace("(anonymous namespace)::", ""))
            if kind is None or r["Counter_Name"] not in counters:
                continue
            v = float(r["Counter_Value"])
            if r["Counter_Name"] in scale:
                v *= 1024 * scale[r["Counter_Name"]]
            acc[kind][r["Counter_Name"]] += v
            if tag == "FETCH_SIZE":
                launches[kind].add(r["Dispatch_Id"])
    kernels = {}
    simds = 1024
    for kind, a in acc.items():
        n = len(launches[kind]) or 1
        k = {"launches": n,
             "hbm_read_bytes_per_launch": round(a.get("FETCH_SIZE", 0) / n),
             "hbm_write_bytes_per_launch": round(a.get("WRITE_SIZE", 0) / n)}
        k["hbm_bytes_per_launch"] = k["hbm_read_bytes_per_launch"] + k["hbm_write_bytes_per_launch"]
        if a.get("TCC_HIT_sum", 0) + a.get("TCC_MISS_sum", 0) > 0:
            k["l2_hit_rate"] = round(a["TCC_HIT_sum"] / (a["TCC_HIT_sum"] + a["TCC_MISS_sum"]), 4)
        if a.get("GRBM_GUI_ACTIVE", 0) > 0:
            k["mfma_busy_fraction"] = round(
                a["SQ_VALU_MFMA_BUSY_CYCLES"] / (a["GRBM_GUI_ACTIVE"] / 8 * simds), 4)
        kernels[kind] = k
    return {"workload": "diffurefill1b_orthogonal_step", "kernel_source_hash": polar_source_hash(),
            "batching": batching,
            "fetch_scale": round(scale.get("FETCH_SIZE", 0), 5),
            "write_scale": round(scale.get("WRITE_SIZE", 0), 5),
            "copy_calibration_bytes": copy_bytes, "command": command, "kernels": kernels}


def polar_pmc_markdown(s: dict) -> str:
    out = ["# Orthogonalisation kernels: counters per dispatch (" + s["workload"] + ")", "",
           "One rocprofv3 --pmc run per counter group, all of the same command; FETCH_SIZE and "
           "WRITE_SIZE (KiB per dispatch) scaled by what the same counter reads for a plain copy "
           f"kernel of {s['copy_calibration_bytes']} bytes: FETCH x{s['fetch_scale']}, "
           f"WRITE x{s['write_scale']}.", "",
           "Command (the counter list after --pmc changes per pass: FETCH_SIZE; WRITE_SIZE; "
           "TCC_HIT_sum TCC_MISS_sum; SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 "
           "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE):", "", "```", s["command"], "```", "",
           f"Kernel source hash: `{s['kernel_source_hash']}`", "",
           "| kind | launches | HBM read / launch (MB) | HBM write / launch (MB) | L2 hit rate | "
           "MFMA busy (of SIMD cycles) |", "|---|---:|---:|---:|---:|---:|"]
    for kind, k in sorted(s["kernels"].items()):
        out.append(f"| {kind} | {k['launches']} | {k['hbm_read_bytes_per_launch'] / 1e6:.1f} | "
                   f"{k['hbm_write_bytes_per_launch'] / 1e6:.1f} | {k.get('l2_hit_rate', 'n/a')} | "
                   f"{k.get('mfma_busy_fraction', 'n/a')} |")
    return "\n".join(out) + "\n"


def stats_markdown(stats_csv: str, command: str, title: str = "Merge kernels") -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}: dispatch durations (rocprofv3 --kernel-trace --stats)", "",
           "Command:", "", "```", command, "```", "",
           "| kind | kernel | calls | average (us) | min (us) | max (us) | total (ms) |",
           "|---|---|---:|---:|---:|---:|---:|"]
    other_calls, other_ns = 0, 0.0
    def col(r, *names):
        low = {k.lower(): v for k, v in r.items()}
        for n in names:
            v = low.get(n.lower())
            if v not in (None, ""):
                return float(v)
        raise KeyError(names)

    for r in rows:
        r = {k.strip(): v for k, v in r.items()}
        name = r.get("Name") or r.get("KernelName") or ""
        calls = int(col(r, "Calls"))
        total = col(r, "TotalDurationNs", "DURATION (nsec)")
        kind = kernel_kind(name)
        if kind is None:
            other_calls += calls
            other_ns += total
            continue
        short = name.replace("void ", "").replace("dlk::(anonymous namespace)::", "")
        short = re.sub(r"\(.*", "", short)
        avg = col(r, "AverageNs", "AVERAGE (nsec)")
        mn = col(r, "MinNs", "MIN (nsec)")
        mx = col(r, "MaxNs", "MAX (nsec)")
        out.append(f"| {kind} | `{short}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                   f"{mx / 1e3:.1f} | {total / 1e6:.2f} |")
    out += ["", f"Other kernels in the same run (input generation): {other_calls} dispatches, "
            f"{other_ns / 1e6:.1f} ms in total.", ""]
    return "\n".join(out)


def _read_pmc(path: str, counter: str):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    return rows


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, cmd_fetch: str, cmd_write: str,
                copy_bytes: int):
    fetch = _read_pmc(fetch_csv, "FETCH_SIZE")
    write = _read_pmc(write_csv, "WRITE_SIZE")
    # calibration: the plain copy kernel of known size (1 read + 1 write of nb bytes)
    def copy_row(rows):
        c = [r for r in rows if "plain_copy" in r["Kernel_Name"]]
        if len(c) != 1:
            raise SystemExit("expected exactly one plain_copy dispatch")
        return c[0]
    f_scale = copy_bytes / (float(copy_row(fetch)["Counter_Value"]) * 1024)
    w_scale = copy_bytes / (float(copy_row(write)["Counter_Value"]) * 1024)
    per = defaultdict(lambda: {"launches": 0, "fetch": 0.0, "write": 0.0, "elements": 0})
    for r in fetch:
        kind = kernel_kind(r["Kernel_Name"])
        if kind is None:
            continue
        d = per[kind]
        d["launches"] += 1
        d["fetch"] += float(r["Counter_Value"]) * 1024 * f_scale
    for r in write:
        kind = kernel_kind(r["Kernel_Name"])
        if kind is None:
            continue
        per[kind]["write"] += float(r["Counter_Value"]) * 1024 * w_scale
    kernels = {}
    for kind, d in per.items():
        kernels[kind] = {
            "launches": d["launches"],
            "hbm_read_bytes_per_launch": round(d["fetch"] / d["launches"]),
            "hbm_write_bytes_per_launch": round(d["write"] / d["launches"]),
            "hbm_bytes_per_launch": round((d["fetch"] + d["write"]) / d["launches"]),
        }
    return {
        "workload": workload,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_scale": round(f_scale, 5),
        "write_scale": round(w_scale, 5),
        "copy_calibration_bytes": copy_bytes,
        "command_fetch": cmd_fetch,
        "command_write": cmd_write,
        "kernels": kernels,
    }


def pmc_markdown(s: dict, alg_per_elem: dict, frag_elems: dict) -> str:
    title = ("Side averages and adoption" if s["workload"] == SIDE_WORKLOAD else "Merge kernels")
    out = [f"# {title}: HBM traffic per dispatch ({s['workload']})", "",
           "FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each from its own rocprofv3 run, "
           "scaled by what the same counter reads for a plain copy kernel of "
           f"{s['copy_calibration_bytes']} bytes: FETCH x{s['fetch_scale']}, "
           f"WRITE x{s['write_scale']}.", "",
           "Commands:", "", "```", s["command_fetch"], s["command_write"], "```", "",
           f"Kernel source hash: `{s['kernel_source_hash']}`", "",
           "| kind | launches | HBM read / launch (GB) | HBM write / launch (GB) | "
           "algorithmic / launch (GB) | measured / algorithmic |",
           "|---|---:|---:|---:|---:|---:|"]
    for kind, k in sorted(s["kernels"].items()):
        alg = alg_per_elem.get(kind.replace("_bf16", ""), 0) * frag_elems.get(kind, 0)
        ratio = f"{k['hbm_bytes_per_launch'] / alg:.4f}" if alg else "n/a"
        out.append(f"| {kind} | {k['launches']} | {k['hbm_read_bytes_per_launch'] / 1e9:.4f} | "
                   f"{k['hbm_write_bytes_per_launch'] / 1e9:.4f} | {alg / 1e9:.4f} | {ratio} |")
    return "\n".join(out) + "\n"


# Raw request counters of the L2-to-memory interface, which need no
# copy-kernel scale: a read counted in 32-byte units towards DRAM (a 64-byte
# request counts 2, a 128-byte one 4), the request counts FETCH_SIZE is
# built from, and the write requests with their 64-byte share and the part
# destined for DRAM.
DRAM_READ_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                      "TCC_BUBBLE_sum")
DRAM_WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum")


def _per_dispatch(path: str, counters):
    """{dispatch id: (kernel name, {counter: value})} of one --pmc pass."""
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in counters:
            continue
        name, vals = out.setdefault(r["Dispatch_Id"], (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def dram_pmc_summary(read_csv: str, write_csv: str, workload: str, cmd_read: str,
                     cmd_write: str) -> dict:
    """Per kernel kind and dispatch: DRAM read bytes from the 32-byte-unit
    counter; the bytes FETCH_SIZE's formula gives from the same pass's
    request counts (128 B per TCC_BUBBLE, 32 B per 32-byte request, 64 B per
    other request), unscaled; write bytes from the write requests (64 B per
    64-byte request, 32 B per other); the share of write requests that go to
    DRAM."""
    reads = _per_dispatch(read_csv, DRAM_READ_COUNTERS)
    writes = _per_dispatch(write_csv, DRAM_WRITE_COUNTERS)
    per = defaultdict(lambda: defaultdict(float))
    for name, v in reads.values():
        kind = kernel_kind(name)
        if kind is None:
            continue
        d = per[kind]
        d["launches"] += 1
        d["dram_read"] += 32 * v.get("TCC_EA0_RDREQ_DRAM_32B_sum", 0.0)
        bubble = v.get("TCC_BUBBLE_sum", 0.0)
        r32 = v.get("TCC_EA0_RDREQ_32B_sum", 0.0)
        rall = v.get("TCC_EA0_RDREQ_sum", 0.0)
        d["fetch_formula"] += 128 * bubble + 64 * (rall - bubble - r32) + 32 * r32
        d["read_requests"] += rall
    for name, v in writes.values():
        kind = kernel_kind(name)
        if kind is None:
            continue
        d = per[kind]
        d["write_launches"] += 1
        w64 = v.get("TCC_EA0_WRREQ_64B_sum", 0.0)
        wall = v.get("TCC_EA0_WRREQ_sum", 0.0)
        d["write"] += 64 * w64 + 32 * (wall - w64)
        d["write_requests"] += wall
        d["write_requests_dram"] += v.get("TCC_EA0_WRREQ_DRAM_sum", 0.0)
    kernels = {}
    for kind, d in per.items():
        n, nw = d["launches"] or 1, d["write_launches"] or 1
        kernels[kind] = {
            "launches": int(d["launches"]),
            "dram_read_bytes_per_launch": round(d["dram_read"] / n),
            "fetch_formula_bytes_per_launch": round(d["fetch_formula"] / n),
            "read_bytes_per_request": (round(d["dram_read"] / d["read_requests"], 2)
                                       if d["read_requests"] else None),
            "write_bytes_per_launch": round(d["write"] / nw),
            "write_requests_to_dram": (round(d["write_requests_dram"] / d["write_requests"], 4)
                                       if d["write_requests"] else None),
        }
    return {"workload": workload, "kernel_source_hash": kernel_source_hash(),
            "command_read": cmd_read, "command_write": cmd_write, "kernels": kernels}


def dram_pmc_markdown(s: dict, alg_per_elem: dict, frag_elems: dict) -> str:
    out = [f"# Merge kernels: DRAM traffic per dispatch from raw request counters "
           f"({s['workload']})", "",
           "Two rocprofv3 --pmc passes of the same command, no copy-kernel calibration:",
           "- reads: TCC_EA0_RDREQ_DRAM_32B (32-byte units, a 128-byte request counted 4) x 32 B,"
           " beside the FETCH_SIZE formula over the same pass's TCC_EA0_RDREQ, "
           "TCC_EA0_RDREQ_32B and TCC_BUBBLE (unscaled);",
           "- writes: 64 B per TCC_EA0_WRREQ_64B + 32 B per other TCC_EA0_WRREQ, and the share "
           "of write requests counted towards DRAM (TCC_EA0_WRREQ_DRAM).", "",
           "Commands:", "", "```", s["command_read"], s["command_write"], "```", "",
           f"Kernel source hash: `{s['kernel_source_hash']}`", "",
           "| kind | launches | DRAM read / launch (GB) | FETCH_SIZE formula / launch (GB) | "
           "read bytes per request | write / launch (GB) | writes to DRAM | "
           "algorithmic / launch (GB) | (read + write) / algorithmic |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for kind, k in sorted(s["kernels"].items()):
        alg = alg_per_elem.get(kind.replace("_bf16", ""), 0) * frag_elems.get(kind, 0)
        tot = k["dram_read_bytes_per_launch"] + k["write_bytes_per_launch"]
        ratio = f"{tot / alg:.4f}" if alg else "n/a"
        out.append(f"| {kind} | {k['launches']} | {k['dram_read_bytes_per_launch'] / 1e9:.4f} | "
                   f"{k['fetch_formula_bytes_per_launch'] / 1e9:.4f} | "
                   f"{k['read_bytes_per_request']} | {k['write_bytes_per_launch'] / 1e9:.4f} | "
                   f"{k['write_requests_to_dram']} | {alg / 1e9:.4f} | {ratio} |")
    return "\n".join(out) + "\n"


def _workload_bytes(key: str, kinds):
    from . import synth
    from .workload import algorithmic_bytes
    if key == SIDE_WORKLOAD:
        # every side-average call runs over the whole DiffuRefill-1B buffer
        return dict(SIDE_BYTES_PER_ELEM), {k: synth.DIFFUREFILL_1B.n_params for k in kinds}
    w = synth.WORKLOADS[key]
    sizes = [w.frag_offsets[f + 1] - w.frag_offsets[f] for f in range(w.n_frags)]
    avg = sum(sizes) / len(sizes)
    return algorithmic_bytes(w)["per_elem"], {k: avg for k in kinds}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("stats_csv")
    a.add_argument("--command", required=True)
    a.add_argument("--title", default="Merge kernels")
    b = sub.add_parser("pmc")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--workload", required=True)
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    b.add_argument("--copy-bytes", type=int, required=True,
                   help="bytes the plain copy kernel read (and wrote)")
    b.add_argument("--json")
    c = sub.add_parser("polar-stats")
    c.add_argument("stats_csv")
    c.add_argument("--command", required=True)
    d = sub.add_parser("polar-pmc")
    d.add_argument("run_dir")
    d.add_argument("--command", required=True)
    d.add_argument("--copy-bytes", type=int, required=True)
    d.add_argument("--json")
    e = sub.add_parser("pmc-dram")
    e.add_argument("read_csv")
    e.add_argument("write_csv")
    e.add_argument("--workload", required=True)
    e.add_argument("--command-read", required=True)
    e.add_argument("--command-write", required=True)
    e.add_argument("--json")
    d.add_argument("--batching", default="even",
                   help="how the run batched equally shaped matrices: 'even' (all of a shape, "
                        "split evenly into launches of at most 64) or the fixed batch size")
    args = ap.parse_args(argv)
    if args.mode == "polar-stats":
        print(polar_stats_markdown(args.stats_csv, args.command))
        return
    if args.mode == "polar-pmc":
        s = polar_pmc_summary(args.run_dir, args.command, args.copy_bytes, args.batching)
        if args.json:
            with open(args.json, "w") as fh:
                json.dump(s, fh, indent=1)
        sys.stdout.write(polar_pmc_markdown(s))
        return
    if args.mode == "stats":
        print(stats_markdown(args.stats_csv, args.command, args.title))
        return
    if args.mode == "pmc-dram":
        s = dram_pmc_summary(args.read_csv, args.write_csv, args.workload, args.command_read,
                             args.command_write)
        if args.json:
            with open(args.json, "w") as fh:
                json.dump(s, fh, indent=1)
        sys.stdout.write(dram_pmc_markdown(s, *_workload_bytes(args.workload, s["kernels"])))
        return
    s = pmc_summary(args.fetch_csv, args.write_csv, args.workload, args.command_fetch,
                    args.command_write, args.copy_bytes)
    from . import synth
    if args.workload == SIDE_WORKLOAD:
        # every side-average call runs over the whole DiffuRefill-1B buffer
        alg = dict(SIDE_BYTES_PER_ELEM)
        frag_elems = {k: synth.DIFFUREFILL_1B.n_params for k in s["kernels"]}
    else:
        from .workload import algorithmic_bytes
        w = synth.WORKLOADS[args.workload]
        alg = algorithmic_bytes(w)["per_elem"]
        # average elements per launch of each kind over the round (all fragments)
        sizes = [w.frag_offsets[f + 1] - w.frag_offsets[f] for f in range(w.n_frags)]
        avg = sum(sizes) / len(sizes)
        frag_elems = {k: avg for k in s["kernels"]}
    if args.json:
        with open(args.json, "w") as fh:
            json.dump(s, fh, indent=1)
    sys.stdout.write(pmc_markdown(s, alg, frag_elems))


if __name__ == "__main__":
    main()
