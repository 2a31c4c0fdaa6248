"""Host-side logic of bench.py: counter CSV parsing, calibration scaling and
the guard that drops stored traffic taken on other kernel sources."""
from __future__ import annotations

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for did, name, val in rows:
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": val})


class _Stub:
    def __init__(self):
        self.launches = [bench.Launch("quant_act_1x128", None, 3000.0),
                         bench.Launch("gemm", None, 10000.0, 1.0)]


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    probe_mib = 1
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    # the copy reads 1 MiB but the fetch counter shows half of it (KiB units)
    _write(fetch, "FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", 512.0),
                                 (2, "void fp8q::quant_act_1x128_kernel<false>(...)", 1.0),
                                 (3, "void fp8q::gemm_kernel<256>(Params)", 4.0),
                                 (4, "void fp8q::gemm_kernel<256>(Params)", 6.0),
                                 (5, "at::native::other", 99.0)])
    _write(write, "WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", 1024.0),
                                 (2, "void fp8q::quant_act_1x128_kernel<false>(...)", 2.0),
                                 (3, "void fp8q::gemm_kernel<256>(Params)", 3.0),
                                 (4, "void fp8q::gemm_kernel<256>(Params)", 3.0)])
    out = str(tmp_path / "t.json")
    res = bench.pmc_summary(fetch, write, "dense_fprop", probe_mib, out, _Stub())
    assert res["fetch_factor"] == 2.0 and res["write_factor"] == 1.0
    g = res["kernels"]["gemm"]
    assert g["fetch_bytes"] == 5 * 1024 * 2 and g["write_bytes"] == 3 * 1024
    assert g["traffic_bytes"] == 13 * 1024 and g["dispatches"] == 2
    assert g["algorithmic_bytes"] == 10000
    q = res["kernels"]["quant_act_1x128"]
    assert q["traffic_bytes"] == 1 * 2048 + 2 * 1024
    with open(out) as f:
        assert json.load(f)["dense_fprop"]["kernel_source"] == bench.kernel_source_digest()
    assert bench.stored_traffic(out, "dense_fprop")["gemm"]["traffic_bytes"] == 13 * 1024


def test_stored_traffic_dropped_for_other_kernel_source(tmp_path):
    out = str(tmp_path / "t.json")
    with open(out, "w") as f:
        json.dump({"dense_fprop": {"kernel_source": "0" * 16, "kernels": {"gemm": {}}}}, f)
    assert bench.stored_traffic(out, "dense_fprop") is None
    assert bench.stored_traffic(out, "wgrad") is None
    assert bench.stored_traffic(str(tmp_path / "missing.json"), "dense_fprop") is None


def test_multi_gpu_request_exits_with_message(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    else:
        raise AssertionError("bench.main() accepted --gpus 2")
    assert "one GPU" in capsys.readouterr().err


def test_pmc_summary_ignores_kernels_outside_the_step(tmp_path):
    """Set-up dispatches (say the 1x128 quantizer making an FP8 cache) whose
    label is not one of the step's launches are not summarized."""
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _write(fetch, "FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", 1024.0),
                                 (2, "void fp8q::quant_act_1x128_kernel<false>(...)", 9.0),
                                 (3, "void fp8q::gemm_kernel<256>(Params)", 4.0)])
    _write(write, "WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", 1024.0),
                                 (2, "void fp8q::quant_act_1x128_kernel<false>(...)", 9.0),
                                 (3, "void fp8q::gemm_kernel<256>(Params)", 3.0)])

    class OnlyGemm:
        launches = [bench.Launch("gemm", None, 100.0, 1.0)]
    res = bench.pmc_summary(fetch, write, "x", 1, str(tmp_path / "t.json"), OnlyGemm())
    assert set(res["kernels"]) == {"gemm"}


def test_kernel_source_digest_ignores_comments_only(tmp_path):
    """Counter figures stay valid across comment edits, not across code edits."""
    a, b, c = tmp_path / "a", tmp_path / "b", tmp_path / "c"
    for d in (a, b, c):
        d.mkdir()
    (a / "k.hip").write_text("// header\nint f(int x) {\n    return x + 1;  // one\n}\n")
    (b / "k.hip").write_text("/* a longer\n   header */\n\nint f(int x) {\n    return x + 1;\n}\n")
    (c / "k.hip").write_text("// header\nint f(int x) {\n    return x + 2;  // one\n}\n")
    assert bench.kernel_source_digest(str(a)) == bench.kernel_source_digest(str(b))
    assert bench.kernel_source_digest(str(a)) != bench.kernel_source_digest(str(c))
    # host-side argument checks are not kernel code
    (a / "api.cpp").write_text("int check(int n) { return n > 0; }\n")
    assert bench.kernel_source_digest(str(a)) == bench.kernel_source_digest(str(b))


def test_cpu_baseline_extras_report_model_and_one_thread_tiny():
    """The oracle timing names the host CPU and times the Tiny step on one
    thread, leaving the thread pools as they were afterwards."""
    from threadpoolctl import threadpool_info
    bench.tiny_one_thread(min_seconds=0.0)  # loads the oracle's pools before they are recorded
    before = sorted((p["user_api"], p["num_threads"]) for p in threadpool_info())
    assert bench.cpu_model()
    r = bench.tiny_one_thread(min_seconds=0.05)
    assert r["threads"] == 1 and r["steps"] >= 1 and r["ms_per_step"] > 0 and r["gflops"] > 0
    assert sorted((p["user_api"], p["num_threads"]) for p in threadpool_info()) == before


def test_counter_table_means_and_derived_columns(tmp_path):
    """Per step kernel: means over its dispatches, MFMA busy at the peak clock
    and the s_waitcnt share; kernels outside the step are left out."""
    p = tmp_path / "c.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    rows = []
    for did, name, t in ((1, "copyBuffer", 1000), (2, "void fp8q::gemm_kernel<256>(...)", 100000),
                         (3, "void fp8q::gemm_kernel<256>(...)", 100000)):
        for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 2.4e9 * 100e-6 / 2), ("SQ_WAIT_INST_ANY", 30.0),
                     ("SQ_WAVE_CYCLES", 120.0)):
            rows.append([did, name, c, v, 0, t])
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)

    class W:
        launches = [bench.Launch("gemm", None, 1.0)]
    table = bench.counter_table(str(p), W()).splitlines()
    assert len(table) == 3 and table[2].startswith("| gemm | 2 | 100.00 |")
    assert table[2].rstrip(" |").endswith("0.500 | 0.250")


def test_pmc_summary_counts_the_fixup_kernel_in_the_gemm_launch(tmp_path):
    """A grouped GEMM launch dispatches gemm_kernel and then the split-K
    fix-up kernel: its per-launch traffic is the average of each kernel's
    dispatches added together, and both count as dispatches of the launch."""
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _write(fetch, "FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", 512.0),
                                 (2, "void fp8q::gemm_kernel<256, false, false, 1>(Params)", 10.0),
                                 (3, "void fp8q::grouped_fixup_kernel<false>(Params)", 2.0),
                                 (4, "void fp8q::gemm_kernel<256, false, false, 1>(Params)", 14.0),
                                 (5, "void fp8q::grouped_fixup_kernel<false>(Params)", 4.0)])
    _write(write, "WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", 1024.0),
                                 (2, "void fp8q::gemm_kernel<256, false, false, 1>(Params)", 5.0),
                                 (3, "void fp8q::grouped_fixup_kernel<false>(Params)", 1.0),
                                 (4, "void fp8q::gemm_kernel<256, false, false, 1>(Params)", 5.0),
                                 (5, "void fp8q::grouped_fixup_kernel<false>(Params)", 1.0)])
    res = bench.pmc_summary(fetch, write, "grouped_fprop", 1, str(tmp_path / "t.json"), _Stub())
    g = res["kernels"]["gemm"]
    assert g["fetch_bytes"] == (12 + 3) * 1024 * 2     # averages 12 and 3 KiB, factor 2
    assert g["write_bytes"] == (5 + 1) * 1024
    assert g["dispatches"] == 4


def test_counter_table_gives_the_fixup_kernel_its_own_row(tmp_path):
    path = str(tmp_path / "c.csv")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for did, name, ns in ((1, "void fp8q::gemm_kernel<256>(Params)", 300000),
                              (2, "void fp8q::grouped_fixup_kernel<false>(Params)", 15000)):
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "SQ_WAVES",
                        "Counter_Value": 8.0, "Start_Timestamp": 0, "End_Timestamp": ns})
    table = bench.counter_table(path, _Stub())
    rows = [l for l in table.splitlines() if l.startswith("| gemm")]
    assert rows[0].startswith("| gemm | 1 | 300.00")
    assert rows[1].startswith("| gemm: grouped_fixup_kernel | 1 | 15.00")
