"""Text summaries of rocprofv3 output for this library's kernels.

Kernel trace (durations)::

    rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o NAME -- python3 bench.py ...
    python -m fp8_quantize_pack_amd.profiling trace DIR/NAME_kernel_stats.csv OUT.txt --command "..."

HBM traffic (two counter runs, one counter each, of the same bench command
with ``--calibrate-copy``)::

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR_F -o fetch -- python3 bench.py ... --calibrate-copy
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR_W -o write -- python3 bench.py ... --calibrate-copy
    python -m fp8_quantize_pack_amd.profiling traffic DIR_F/fetch_counter_collection.csv \\
        DIR_W/write_counter_collection.csv OUT.txt --copy-bytes N --command-fetch "..." --command-write "..."

FETCH_SIZE and WRITE_SIZE are KiB per dispatch.  Each is scaled by the
factor that maps the same counter, read on the calibration kernel (a torch
elementwise negation that reads N bytes and writes N bytes), to N: the
traffic of a kernel is fetch * 1024 * f_fetch + write * 1024 * f_write bytes
per launch, averaged over its dispatches.  The traffic file names the hash of
the kernel sources it was taken on; bench.py uses it only while the sources
are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))

# bench.py operation -> kernel (bfloat16 instantiations of the launched
# templates for the shapes bench.py runs)
BENCH_KERNELS = {
    "mxfp4_quant": "mxq::k_mxfp4_quant<1>",
    "mxfp4_dequant": "mxq::k_mxfp4_dequant<1>",
    "nvfp4_quant": "mxq::k_nvfp4_quant_seg<1, 7, 1, true>",
    "nvfp4_dequant": "mxq::k_nvfp4_dequant_seg<1>",
    "cache_fp8": "mxq::k_cache_qdq<1, 0, 32>",
    "cache_mxfp4": "mxq::k_cache_qdq<1, 1, 32>",
    "cache_nvfp4": "mxq::k_cache_qdq<1, 2, 16>",
    "nvfp4_tensor_amax": "mxq::k_tensor_amax<1>",
    "nvfp4_quant_tensor_mode": "mxq::k_nvfp4_quant_seg<1, 4, 1, true>",
    "mxfp8_quant": "mxq::k_mxfp8_quant<1>",
    "mxfp8_dequant": "mxq::k_mxfp8_dequant<1>",
    "fp4_static_qdq": "mxq::k_fp4_static_qdq<1>",
    "kv_head_amax": "mxq::k_kv_head_amax<1, true, 16>",
    "kv_quant": "mxq::k_kv_quant<1, true, 16>",
    "kv_pages_dequant": "mxq::k_kv_pages_dequant<1>",
    "gemm_mxfp4_forward": "mxq::gmm::k_grouped_mm<1, 0, 128>",
    "gemm_mxfp4_backward": "mxq::gmm::k_grouped_mm<1, 1, 128>",
    "gemm_nvfp4_forward": "mxq::gmm::k_grouped_mm<2, 0, 128>",
    "gemm_nvfp4_backward": "mxq::gmm::k_grouped_mm<2, 1, 128>",
}
CALIBRATION_MARK = "neg_kernel"


# the sources that decide what the codec kernels bench.py measures execute
# (device code, its headers and the launchers; names and contents hashed).
# Host-side argument checking does not change a kernel's traffic.
CODEC_SOURCES = ("mxq_device.h", "mxq_kernel_common.h", "mxq_nvfp4_common.h",
                 "k_mxfp4.hip", "k_nvfp4.hip", "k_cache.hip",
                 "k_mxfp8.hip", "k_fp4_static.hip", "k_kv.hip")


def code_tokens(text: str) -> str:
    """C/C++/HIP source with comments removed and runs of whitespace folded:
    what the compiler sees, so comment-only edits keep a measurement valid."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":                       # string / char literal, kept verbatim
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the codec kernel sources under csrc/ (code only, see code_tokens)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in CODEC_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def summarize_trace(stats_csv: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [
        "# rocprofv3 kernel trace of bench.py (one MI355X): per-kernel launch durations",
        f"# command: {command}",
        f"# kernel_source_hash: {kernel_source_hash()}",
        "# durations in microseconds over all dispatches (the sweep's last chunk holds 4 experts, the others 36)",
        f"{'op':20s} {'kernel':42s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}",
    ]
    by_kernel = {short_name(r["Name"]): r for r in rows}
    for op, k in BENCH_KERNELS.items():
        r = by_kernel.get(k)
        if r is None:
            continue
        out.append(f"{op:20s} {k:42s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    others = [short_name(r["Name"]) for r in rows if short_name(r["Name"]) not in BENCH_KERNELS.values()]
    if others:
        out.append("# other kernels in the process (input generation, torch): " + ", ".join(sorted(set(o[:60] for o in others))))
    return "\n".join(out) + "\n"


def _counter_means(path: str, counter: str):
    """Mean counter value per dispatch, by kernel."""
    acc = defaultdict(lambda: [0.0, 0])
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        acc[k][0] += float(r["Counter_Value"])
        acc[k][1] += 1
    return {k: (s / n, n) for k, (s, n) in acc.items()}


def summarize_traffic(fetch_csv: str, write_csv: str, copy_bytes: int,
                      cmd_fetch: str, cmd_write: str, algorithmic: dict) -> str:
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    cal_f = [v for k, v in fetch.items() if CALIBRATION_MARK in k]
    cal_w = [v for k, v in write.items() if CALIBRATION_MARK in k]
    if not cal_f or not cal_w:
        raise SystemExit("calibration kernel not found in the counter files (run bench.py with --calibrate-copy)")
    f_fetch = copy_bytes / (cal_f[0][0] * 1024.0)
    f_write = copy_bytes / (cal_w[0][0] * 1024.0)
    out = [
        "# HBM traffic per launch from rocprofv3 counters (one MI355X)",
        f"# command (fetch): {cmd_fetch}",
        f"# command (write): {cmd_write}",
        f"source_hash: {kernel_source_hash()}",
        f"# calibration: torch neg over {copy_bytes} bytes read + {copy_bytes} bytes written reads "
        f"FETCH_SIZE {cal_f[0][0]:.0f} KiB (factor {f_fetch:.4f}), WRITE_SIZE {cal_w[0][0]:.0f} KiB (factor {f_write:.4f})",
        "# per op: scaled fetch + write bytes per launch (mean over dispatches) vs the algorithmic bytes per launch",
    ]
    for op, k in BENCH_KERNELS.items():
        if k not in fetch or k not in write:
            continue
        fb = fetch[k][0] * 1024.0 * f_fetch
        wb = write[k][0] * 1024.0 * f_write
        alg = algorithmic.get(op)
        ratio = f"  ratio_to_algorithmic: {(fb + wb) / alg:.4f}" if alg else ""
        out.append(f"{op} traffic_bytes_per_launch: {fb + wb:.0f}  fetch: {fb:.0f}  write: {wb:.0f}  "
                   f"dispatches: {fetch[k][1]}{ratio}")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv"); t.add_argument("out"); t.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_csv"); c.add_argument("write_csv"); c.add_argument("out")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command-fetch", required=True); c.add_argument("--command-write", required=True)
    c.add_argument("--algorithmic", default="", help="op=bytes,... algorithmic bytes per launch")
    a = ap.parse_args()
    if a.what == "trace":
        txt = summarize_trace(a.stats_csv, a.command)
    else:
        alg = {}
        for kv in filter(None, a.algorithmic.split(",")):
            k, v = kv.split("=")
            alg[k] = float(v)
        txt = summarize_traffic(a.fetch_csv, a.write_csv, a.copy_bytes, a.command_fetch, a.command_write, alg)
    with open(a.out, "w") as f:
        f.write(txt)
    print(txt, end="")


if __name__ == "__main__":
    main()
