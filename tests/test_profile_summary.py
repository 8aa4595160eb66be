"""Host checks of the counter and trace summaries: kernel kinds from
demangled names, the copy-calibrated byte counts, and the committed HBM
traffic summaries against the algorithmic bytes of each kernel."""
import csv
import json
import os

import pytest

from checkpoint_averaging_amd import profile_summary as ps
from checkpoint_averaging_amd import synth
from checkpoint_averaging_amd.workload import algorithmic_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,kind", [
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldSum<float, true>, true>"
     "(dlk::(anonymous namespace)::FoldSum<float, true>, long, int)", "fold_first"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldSum<unsigned short, "
     "false>, true>(...)", "fold_bf16"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldDelta<float, false>, "
     "true>(...)", "fold_delta"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldNesterovClose<float, "
     "false, true>, true>(...)", "fold_nesterov_ema"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::MeanClose<false>, true>(...)",
     "finalize_mean"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::SnapshotMean<5>, true>(...)",
     "snapshot_mean_5"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::AdoptKeepDrift<float>, "
     "true>(...)", "adopt_keep_drift"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldManyNesterovClose<"
     "float, true, true>, true>(...)", "fold_all_nesterov_ema"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldManyMeanClose<"
     "unsigned short, true, true>, true>(...)", "fold_all_finalize_mean_ema_bf16"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldDeltaMany<float, "
     "false>, true>(...)", "fold_delta_all_more"),
    ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldSumMany<float, "
     "true>, false>(...)", "fold_all"),
    ("void at::native::vectorized_elementwise_kernel<4, ...>(...)", None),
])
def test_kernel_kind(name, kind):
    assert ps.kernel_kind(name) == kind


@pytest.mark.parametrize("name,kind", [
    ("void dlk::(anonymous namespace)::k_gemm<true>(float const*, long, ...)", "gemm_TN"),
    ("void dlk::(anonymous namespace)::k_gemm<false>(float const*, long, ...)", "gemm_NT"),
    ("void dlk::(anonymous namespace)::k_gemm_big<true>(float const*, long, ...)", "gemm_big_TN"),
    ("void dlk::(anonymous namespace)::k_gemm_big<false>(float const*, long, ...)",
     "gemm_big_NT"),
    ("dlk::(anonymous namespace)::k_reduce_big(float const*, dlk::(anonymous namespace)::BigWork, "
     "dlk::(anonymous namespace)::Epilogue)", "reduce_big"),
    ("dlk::(anonymous namespace)::k_reduce_splits(float const*, ...)", "reduce_splits"),
    ("dlk::(anonymous namespace)::k_sumsq_partial(dlk::(anonymous namespace)::MatPtrs, ...)",
     "sumsq_partial"),
    ("dlk::(anonymous namespace)::k_step(dlk::(anonymous namespace)::MatPtrsW, ...)", "step"),
    ("void dlk::(anonymous namespace)::k_stream<...FoldSum<float, true>, true>(...)", None),
])
def test_polar_kind(name, kind):
    assert ps.polar_kind(name) == kind


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, val in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path):
    fold = ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldSum<float, "
            "false>, true>(...)")
    nb = 1 << 30
    # the fetch counter reads half of what is moved, the write counter all of it
    _write_csv(tmp_path / "f.csv", "FETCH_SIZE",
               [("plain_copy(float4 const*, float4*, long)", nb / 2 / 1024),
                (fold, 3 * nb / 2 / 1024), (fold, 3 * nb / 2 / 1024)])
    _write_csv(tmp_path / "w.csv", "WRITE_SIZE",
               [("plain_copy(float4 const*, float4*, long)", nb / 1024), (fold, nb / 1024),
                (fold, nb / 1024)])
    s = ps.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "x", "cf", "cw", nb)
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    k = s["kernels"]["fold"]
    assert k["launches"] == 2
    assert k["hbm_read_bytes_per_launch"] == 3 * nb
    assert k["hbm_bytes_per_launch"] == 4 * nb


def _committed(name):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        pytest.skip(f"{name} not present")
    with open(path) as fh:
        return json.load(fh)


def test_merge_kernels_move_their_algorithmic_bytes():
    d = _committed("pmc_diffurefill1b_frag_nesterov_ema.json")
    w = synth.WORKLOADS[d["workload"]]
    per = algorithmic_bytes(w)["per_elem"]
    avg = w.n_params / w.n_frags
    for kind, k in d["kernels"].items():
        assert k["hbm_bytes_per_launch"] == pytest.approx(per[kind] * avg, rel=5e-3), kind


def test_side_average_kernels_move_their_algorithmic_bytes():
    d = _committed("pmc_diffurefill1b_side_averages.json")
    n = synth.DIFFUREFILL_1B.n_params
    assert set(d["kernels"]) <= set(ps.SIDE_BYTES_PER_ELEM)
    for kind, k in d["kernels"].items():
        assert k["hbm_bytes_per_launch"] == pytest.approx(ps.SIDE_BYTES_PER_ELEM[kind] * n,
                                                          rel=5e-3), kind


def test_source_hash_ignores_comments_only():
    src = ('// header\nint f(int a) { /* inline */ return a + 1; }  // tail\n'
           'const char* s = "http://x /* kept */";\n')
    same = ('/* another header */\nint f(int a) {\n    return a + 1;\n}\n'
            'const char* s = "http://x /* kept */";  // other tail\n')
    code = src.replace("a + 1", "a + 2")
    strip = ps.strip_comments
    assert strip(src) == strip(same)
    assert strip(src) != strip(code)
    assert '"http://x /* kept */"' in strip(src)      # string literals untouched


def test_dram_summary_counts_bytes_from_requests(tmp_path):
    """Raw request counters: 32 B per 32-byte unit of DRAM reads, the
    FETCH_SIZE formula over the request counts, 64 B per 64-byte write
    request and 32 B per other."""
    fold = ("void dlk::(anonymous namespace)::k_stream<dlk::(anonymous namespace)::FoldSum<float, "
            "false>, true>(...)")
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(tmp_path / "r.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for d in ("1", "2"):
            # 1000 read requests of 128 B, seen as TCC_BUBBLE, plus 10 of 32 B
            for c, v in (("TCC_EA0_RDREQ_DRAM_32B_sum", 4 * 1000 + 10),
                         ("TCC_EA0_RDREQ_sum", 1010), ("TCC_EA0_RDREQ_32B_sum", 10),
                         ("TCC_BUBBLE_sum", 1000)):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": fold, "Counter_Name": c,
                            "Counter_Value": v})
        w.writerow({"Dispatch_Id": "3", "Kernel_Name": "other_kernel", "Counter_Name":
                    "TCC_EA0_RDREQ_DRAM_32B_sum", "Counter_Value": 7})
    with open(tmp_path / "w.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for d in ("1", "2"):
            for c, v in (("TCC_EA0_WRREQ_sum", 600), ("TCC_EA0_WRREQ_64B_sum", 500),
                         ("TCC_EA0_WRREQ_DRAM_sum", 600)):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": fold, "Counter_Name": c,
                            "Counter_Value": v})
    s = ps.dram_pmc_summary(str(tmp_path / "r.csv"), str(tmp_path / "w.csv"), "x", "cr", "cw")
    k = s["kernels"]["fold"]
    assert k["launches"] == 2
    assert k["dram_read_bytes_per_launch"] == 32 * 4010
    assert k["fetch_formula_bytes_per_launch"] == 128 * 1000 + 32 * 10
    assert k["read_bytes_per_request"] == pytest.approx(32 * 4010 / 1010, abs=0.01)
    assert k["write_bytes_per_launch"] == 64 * 500 + 32 * 100
    assert k["write_requests_to_dram"] == 1.0
    md = ps.dram_pmc_markdown(s, {"fold": 12}, {"fold": 10})
    assert "| fold | 2 |" in md


@pytest.mark.parametrize("key", ["diffurefill1b_frag_nesterov_ema", "diffurefill1b_mean_ema",
                                 "diffurefill1b_bf16_mean_ema", "diffurefill1b_side_averages",
                                 "diffurefill1b_frag_nesterov_ema_bench"])
def test_raw_dram_counters_match_algorithmic_bytes(key):
    """The committed raw-counter summaries: DRAM reads (32-byte units) plus
    writes equal each kernel's algorithmic bytes with no calibration, and
    FETCH_SIZE's formula over the same requests reads half (every read is a
    128-byte request, which it counts as 64 bytes)."""
    d = _committed(f"dram_traffic_{key}.json")
    if d["workload"] == ps.SIDE_WORKLOAD:
        per, avg = ps.SIDE_BYTES_PER_ELEM, synth.DIFFUREFILL_1B.n_params
    else:
        w = synth.WORKLOADS[d["workload"]]
        per, avg = algorithmic_bytes(w)["per_elem"], w.n_params / w.n_frags
    for kind, k in d["kernels"].items():
        total = k["dram_read_bytes_per_launch"] + k["write_bytes_per_launch"]
        assert total == pytest.approx(per[kind.replace("_bf16", "")] * avg, rel=5e-3), kind
        assert k["fetch_formula_bytes_per_launch"] == pytest.approx(
            k["dram_read_bytes_per_launch"] / 2, rel=1e-3), kind
        assert k["read_bytes_per_request"] == pytest.approx(128.0, rel=1e-3), kind
