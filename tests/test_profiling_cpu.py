"""The rocprofv3 summariser: kernel-trace table and calibrated HBM traffic,
on small hand-written CSV files (no GPU)."""
import csv

from fp8_quantize_pack_amd import profiling as prof

FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_is_scaled_by_the_calibration_kernel(tmp_path):
    n = 1 << 30
    neg = "void (anonymous namespace)::k_copy<2>(unsigned int vector[4] const*, unsigned int vector[4]*, long, long)"
    q = "void mxq::k_nvfp4_quant_seg<1, 7, 1, true>(void const*, mxq::NvSegGeom)"
    # the fetch counter reads half of the true bytes, the write counter all of them
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                    [(neg, n / 2048), (q, 1000.0), (q, 3000.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(neg, n / 1024), (q, 500.0), (q, 500.0)])
    txt = prof.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), n,
                                 "cmd-f", "cmd-w", {"nvfp4_quant": 4608000.0})
    line = [l for l in txt.splitlines() if l.startswith("nvfp4_quant ")][0]
    # fetch: mean 2000 KiB * 1024 * 2; write: 500 KiB * 1024 * 1
    assert "traffic_bytes_per_launch: 4608000 " in line
    assert "fetch: 4096000 " in line and "write: 512000 " in line
    assert "ratio_to_algorithmic: 1.0000" in line
    assert "source_hash: " + prof.kernel_source_hash() in txt


def test_trace_table_maps_bench_ops_to_kernels(tmp_path):
    path = tmp_path / "stats.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void mxq::k_mxfp4_quant<1>(void const*, unsigned int*)", "Calls": 8,
                    "TotalDurationNs": 1600000, "AverageNs": 200000, "Percentage": 50.0,
                    "MinNs": 25000, "MaxNs": 230000})
        w.writerow({"Name": "some_other_kernel", "Calls": 1, "TotalDurationNs": 5,
                    "AverageNs": 5, "Percentage": 0.0, "MinNs": 5, "MaxNs": 5})
    txt = prof.summarize_trace(str(path), "cmd")
    row = [l for l in txt.splitlines() if l.startswith("mxfp4_quant")][0].split()
    assert row[1] == "mxq::k_mxfp4_quant<1>" and row[2] == "8" and row[3] == "200.00"
    assert "some_other_kernel" in txt


def test_code_tokens_ignore_comments_and_layout_only():
    a = "int x = 1; // one\n/* block\n comment */ float y;\nconst char* s = \"// not a comment\";"
    b = "int x = 1;\n\n   float y;   const char* s = \"// not a comment\";"
    assert prof.code_tokens(a) == prof.code_tokens(b)
    assert prof.code_tokens("int x = 1;") != prof.code_tokens("int x = 2;")
    assert "// not a comment" in prof.code_tokens(a)



def test_runs_table_groups_back_to_back_dispatches(tmp_path):
    path = tmp_path / "trace.csv"
    nv = "void mxq::k_nvfp4_quant_seg<1, 7, 1, true>(void const*, mxq::NvSegGeom)"
    mx = "void mxq::k_mxfp4_dequant<1>(unsigned int const*, unsigned char const*)"
    rows, t = [], 0
    for name, n, dur in ((mx, 2, 100), (nv, 3, 200), (mx, 1, 100), (nv, 2, 50), (nv, 0, 0)):
        for _ in range(n):
            rows.append((name, t, t + dur * 1000))
            t += dur * 1000 + 5000
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, a, b in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": a, "End_Timestamp": b})
    txt = prof.summarize_runs(str(path), "cmd", "nvfp4_quant", 3)
    lines = [l for l in txt.splitlines() if not l.startswith("#") and not l.startswith("predecessor")]
    # only the 3-dispatch run counts; its predecessor is the MXFP4 dequantizer, 5 us before it
    assert len(lines) == 1
    f = lines[0].split()
    assert f[0] == "mxfp4_dequant" and f[1] == "5.0" and f[2] == "200.0" and f[5] == "600.0"
