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
factor that maps the same counter, read on the calibration kernel (the
reference copy kernel of libmxq_roofline, which reads N bytes and writes N
bytes), to N: the
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
# templates for the shapes bench.py runs, float16 where the op says so)
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
    "mxfp4_dequant_f16": "mxq::k_mxfp4_dequant<2>",
    "nvfp4_dequant_f16": "mxq::k_nvfp4_dequant_seg<2>",
    "fp4_static_qdq": "mxq::k_fp4_static_qdq<1>",
    "kv_head_amax": "mxq::k_kv_head_amax<1, true, 16>",
    "kv_quant": "mxq::k_kv_quant<1, true, 16>",
    "kv_pages_dequant": "mxq::k_kv_pages_dequant<1>",
    "gemm_mxfp4_forward": "mxq::gmm::k_grouped_mm<1, 0, 256, true>",
    "gemm_mxfp4_backward": "mxq::gmm::k_grouped_mm<1, 1, 256, true>",
    "gemm_nvfp4_forward": "mxq::gmm::k_grouped_mm<2, 0, 256, false>",
    "gemm_nvfp4_backward": "mxq::gmm::k_grouped_mm<2, 1, 256, false>",
    "ref_copy_u1": "(anonymous namespace)::k_copy<1>",
    "ref_copy_u2": "(anonymous namespace)::k_copy<2>",
    "ref_copy_u4": "(anonymous namespace)::k_copy<4>",
    "ref_read_u1": "(anonymous namespace)::k_read<1>",
    "ref_read_u2": "(anonymous namespace)::k_read<2>",
    "ref_read_u4": "(anonymous namespace)::k_read<4>",
    "ref_write_u1": "(anonymous namespace)::k_fill<1>",
    "ref_write_u2": "(anonymous namespace)::k_fill<2>",
    "ref_write_u4": "(anonymous namespace)::k_fill<4>",
}
CALIBRATION_MARK = "k_copy<2>"


# the sources that decide what the codec kernels bench.py measures execute
# (device code, its headers and the launchers; names and contents hashed).
# Host-side argument checking does not change a kernel's traffic.
CODEC_SOURCES = ("mxq_device.h", "mxq_kernel_common.h", "mxq_nvfp4_common.h",
                 "k_mxfp4.hip", "k_nvfp4.hip", "k_cache.hip",
                 "k_mxfp8.hip", "k_fp4_static.hip", "k_kv.hip", "k_grouped_mm.hip")


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
    """Kernel name without its return type and parameter list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    anon = "(anonymous namespace)"
    return name.replace(anon, "\0").split("(")[0].replace("\0", anon)


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


def summarize_trace_dispatches(trace_csv: str, command: str) -> str:
    """Per bench op, its dispatches grouped by grid size (one line per
    size: the sweep's 36- and 4-expert chunks, the cache tensors, and any
    other size the bench launches the same kernel at), from rocprofv3's
    per-dispatch kernel trace."""
    groups = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        k = short_name(r["Kernel_Name"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups[(k, grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [
        "# rocprofv3 kernel trace of bench.py (one MI355X): launch durations per kernel and grid size",
        f"# command: {command}",
        f"# kernel_source_hash: {kernel_source_hash()}",
        "# durations in microseconds; grid = work-items of the dispatch",
        f"{'op':24s} {'grid':>10s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}",
    ]
    for op, k in BENCH_KERNELS.items():
        for (kk, grid), ts in sorted(groups.items(), key=lambda g: -g[0][1]):
            if kk != k:
                continue
            out.append(f"{op:24s} {grid:10d} {len(ts):6d} {sum(ts) / len(ts):9.2f} "
                       f"{min(ts):9.2f} {max(ts):9.2f}")
    return "\n".join(out) + "\n"


def _grid(r) -> int:
    if "Grid_Size" in r:
        return int(float(r["Grid_Size"]))
    return 0


def _counter_means(path: str, counter: str, only_grids=None):
    """Mean counter value per dispatch, by kernel.  only_grids maps a kernel
    to the grid sizes (work-items) whose dispatches count for it (the bench
    launches some kernels at other sizes too)."""
    acc = defaultdict(lambda: [0.0, 0])
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        if only_grids and k in only_grids and _grid(r) not in only_grids[k]:
            continue
        acc[k][0] += float(r["Counter_Value"])
        acc[k][1] += 1
    return {k: (s / n, n) for k, (s, n) in acc.items()}


def summarize_traffic(fetch_csv: str, write_csv: str, copy_bytes: int,
                      cmd_fetch: str, cmd_write: str, algorithmic: dict,
                      only_grids=None) -> str:
    og = {BENCH_KERNELS[op]: g for op, g in (only_grids or {}).items()}
    fetch = _counter_means(fetch_csv, "FETCH_SIZE", og)
    write = _counter_means(write_csv, "WRITE_SIZE", og)
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
        f"# calibration: the reference copy over {copy_bytes} bytes read + {copy_bytes} bytes written reads "
        f"FETCH_SIZE {cal_f[0][0]:.0f} KiB (factor {f_fetch:.4f}), WRITE_SIZE {cal_w[0][0]:.0f} KiB (factor {f_write:.4f})",
        "# per op: scaled fetch + write bytes per launch (mean over dispatches) vs the algorithmic bytes per launch",
    ]
    for op, g in sorted((only_grids or {}).items()):
        out.append(f"# {op}: only dispatches of grid sizes {sorted(g)} (the sweep's chunks)")
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


CU_NUM = 256      # compute units of one MI355X
XCD_NUM = 8       # GRBM_GUI_ACTIVE is reported summed over the XCDs


def summarize_counters(csvs, command: str, elements: dict) -> str:
    """Per bench op: mean per dispatch of every counter in the given
    rocprofv3 --pmc CSV files (one pass each), and the derived
    VALUBusy = 100 * SQ_ACTIVE_INST_VALU / CU_NUM / (GRBM_GUI_ACTIVE / XCD_NUM)
    (rocprof's own formula, with the GPU-busy cycles of one XCD), the VALU
    issue per CU cycle, wave-instructions x 64 lanes per element, and the
    share of wave time spent waiting for any instruction to issue."""
    means = defaultdict(dict)
    for path in csvs:
        acc = defaultdict(lambda: [0.0, 0])
        for r in csv.DictReader(open(path)):
            k = (short_name(r["Kernel_Name"]), r["Counter_Name"])
            acc[k][0] += float(r["Counter_Value"])
            acc[k][1] += 1
        for (k, c), (tot, n) in acc.items():
            means[k][c] = tot / n
    out = [
        "# rocprofv3 counters per dispatch (one MI355X), mean over the op's dispatches",
        f"# command: {command}",
        f"source_hash: {kernel_source_hash()}",
        "# VALUBusy% = 100 * SQ_ACTIVE_INST_VALU / 256 / (GRBM_GUI_ACTIVE / 8); "
        "valu_per_cu_cycle = SQ_INSTS_VALU / 256 / (GRBM_GUI_ACTIVE / 8); "
        "valu_lane_ops_per_elem = 64 * SQ_INSTS_VALU / elements; wait% = 100 * SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
    ]
    for op, k in BENCH_KERNELS.items():
        m = means.get(k)
        if not m:
            continue
        parts = []
        grbm = m.get("GRBM_GUI_ACTIVE")
        if grbm and "SQ_ACTIVE_INST_VALU" in m:
            parts.append(f"VALUBusy%: {100 * m['SQ_ACTIVE_INST_VALU'] / CU_NUM / (grbm / XCD_NUM):.1f}")
        if grbm and "SQ_INSTS_VALU" in m:
            parts.append(f"valu_per_cu_cycle: {m['SQ_INSTS_VALU'] / CU_NUM / (grbm / XCD_NUM):.3f}")
        if op in elements and "SQ_INSTS_VALU" in m:
            parts.append(f"valu_lane_ops_per_elem: {64 * m['SQ_INSTS_VALU'] / elements[op]:.2f}")
        if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES"):
            parts.append(f"wait%: {100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1f}")
        out.append(f"{op} " + "  ".join(parts))
        out.append("    " + "  ".join(f"{c}: {v:.0f}" for c, v in sorted(m.items())))
    return "\n".join(out) + "\n"


def summarize_runs(trace_csv: str, command: str, op: str, length: int) -> str:
    """Runs of `length` back-to-back dispatches of one bench op (a graph
    replay of its chunk launches) in a per-dispatch kernel trace, each with
    the op of the dispatches just before it, the idle gap before the run and
    its per-dispatch durations: how an op's time depends on its predecessor,
    and whether that holds for the whole run or only its first launch."""
    inv = {v: k for k, v in BENCH_KERNELS.items()}
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Kernel_Name"])
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), inv.get(name, name)))
    rows.sort()
    runs, i = [], 0
    while i < len(rows):
        j = i
        while j < len(rows) and rows[j][2] == rows[i][2]:
            j += 1
        runs.append((rows[i][2], i, j))
        i = j
    out = [f"# rocprofv3 kernel trace (one MI355X): runs of {length} back-to-back {op} dispatches and "
           "the op just before each run",
           f"# command: {command}",
           f"# kernel_source_hash: {kernel_source_hash()}",
           "# durations in microseconds; gap = idle time between the predecessor's last dispatch and the run",
           f"{'predecessor':28s} {'gap_us':>7s} {'first':>8s} {'middle_mean':>11s} {'last':>7s} {'run_sum':>8s}"]
    for k, (name, i, j) in enumerate(runs):
        if name != op or j - i != length or k == 0:
            continue
        d = [(rows[t][1] - rows[t][0]) / 1e3 for t in range(i, j)]
        gap = (rows[i][0] - rows[i - 1][1]) / 1e3
        mid = sum(d[1:-1]) / max(1, len(d) - 2)
        out.append(f"{runs[k - 1][0][:28]:28s} {gap:7.1f} {d[0]:8.1f} {mid:11.1f} {d[-1]:7.1f} {sum(d):8.1f}")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv"); t.add_argument("out"); t.add_argument("--command", required=True)
    t.add_argument("--dispatches", default=None,
                   help="the per-dispatch kernel_trace.csv: add durations per grid size")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_csv"); c.add_argument("write_csv"); c.add_argument("out")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command-fetch", required=True); c.add_argument("--command-write", required=True)
    c.add_argument("--algorithmic", default="", help="op=bytes,... algorithmic bytes per launch")
    c.add_argument("--only-grids", default="", help="op=g1:g2,... grid sizes that count for op")
    q = sub.add_parser("counters")
    q.add_argument("out"); q.add_argument("csvs", nargs="+")
    q.add_argument("--command", required=True)
    q.add_argument("--elements", default="", help="op=elements,... elements per launch")
    r = sub.add_parser("runs")
    r.add_argument("trace_csv"); r.add_argument("out"); r.add_argument("--command", required=True)
    r.add_argument("--op", required=True); r.add_argument("--length", type=int, default=8)
    a = ap.parse_args()
    if a.what == "runs":
        txt = summarize_runs(a.trace_csv, a.command, a.op, a.length)
    elif a.what == "trace":
        txt = summarize_trace(a.stats_csv, a.command)
        if a.dispatches:
            txt += "\n" + summarize_trace_dispatches(a.dispatches, a.command)
    elif a.what == "counters":
        el = {}
        for kv in filter(None, a.elements.split(",")):
            k, v = kv.split("=")
            el[k] = float(v)
        txt = summarize_counters(a.csvs, a.command, el)
    else:
        alg = {}
        for kv in filter(None, a.algorithmic.split(",")):
            k, v = kv.split("=")
            alg[k] = float(v)
        og = {}
        for kv in filter(None, a.only_grids.split(",")):
            k, v = kv.split("=")
            og[k] = {int(x) for x in v.split(":")}
        txt = summarize_traffic(a.fetch_csv, a.write_csv, a.copy_bytes, a.command_fetch,
                                a.command_write, alg, og)
    with open(a.out, "w") as f:
        f.write(txt)
    print(txt, end="")


if __name__ == "__main__":
    main()
